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

#include <vector>

#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "decode_mfma.h"
#include "partition.h"
#include "pop_device.h"
#include "pop_internal.h"

namespace pop {

// Channel of gate/up position p: R[p] for p < n_R, then C[p - n_R];
// identity when R is NULL (dense).
// Channel ids read from caller lists are clamped into [0, d_ff): an invalid
// list gives a wrong result, never an out-of-bounds read.
__device__ __forceinline__ int clamp_channel(int ch, int d_ff) { return min(max(ch, 0), d_ff - 1); }

__device__ __forceinline__ int gateup_channel(const int32_t* R, int n_R, const int32_t* C, int p, int d_ff) {
  return clamp_channel(p < n_R ? R[p] : C[p - n_R], d_ff);
}

// ---------------------------------------------------------------- K4
// Block: 256 threads = 4 waves; one gate/up row pair per wave at a time.
// Each lane reads 16-byte vectors of the gate and up rows (two rows, U
// vectors each in flight) and the matching vectors of x (cache-resident).
// BT batch rows are accumulated per pass over the weights.
// kIdentity: rows 0..n_R-1 in order (the dense baseline); a separate
// instantiation so profiles tell the dense and pruned kernels apart.
template <typename T, int BT, bool kIdentity>
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
    const int ch = kIdentity ? p : gateup_channel(R, n_R, C, p, d_ff);
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
// The candidate top-k as its own one-workgroup launch (topk_select; dynamic
// LDS topk_lds_bytes<kTopkThreads>(n)).
constexpr int kTopkThreads = 1024;

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ score, int n, int k,
                                                       const int32_t* __restrict__ C, int32_t* __restrict__ positions,
                                                       int32_t* __restrict__ selected) {
  extern __shared__ __align__(16) unsigned char topk_smem[];
  topk_select<kTopkThreads>(score, n, k, C, positions, selected, topk_smem);
}

// ---------------------------------------------------------------- fused decode step (batch 1)
// Row streaming at batch 1.  A block of 256 threads works on one row at a time
// together: thread t owns the columns j*256*V + t*V + [0, V) (j < NV) of every
// row, so a row's gate, up and W_downT vectors are 3*NV 16-byte loads per
// thread.  Rows go in batches of two, double-buffered: the next batch's loads
// are in flight while the current batch's dot products are reduced (DPP
// within each wave, LDS across the four waves, fixed order).
// A decode step is two launches of k_pop_step and one of k_pop_finish.  Each
// k_pop_step launch gives its first blocks to a link of the candidate chain and
// the rest to a share of the retained rows (gate, up and W_downT rows: z and a
// partial y per block), so the chain's links run beside retained work instead
// of alone:
//   phase 1: candidate rows (z and scores)            + retained share A
//   phase 2: the top-k over those scores (one block)  + retained share B
// k_pop_finish then owns y: each block takes a slice of columns and adds, in a
// fixed order, every retained partial and the selected rows' z * W_downT.  No
// block waits on another inside a launch: each link reads what an earlier
// launch wrote.
// Launch-shape tunables (overridable with -D for sweeps).
#ifndef POP_FUSED_RBLOCKS
#define POP_FUSED_RBLOCKS 256  // most blocks for the retained rows (one per CU)
#endif
#ifndef POP_FUSED_CROWS
#define POP_FUSED_CROWS 4  // candidate rows per block
#endif
#ifndef POP_SPLIT_B
#define POP_SPLIT_B 100  // percent of the retained blocks beside the top-k
#endif
#ifndef POP_FIN_COLS
#define POP_FIN_COLS 32  // columns of y per k_pop_finish block (16, 32 or 64)
#endif
// Retained partial sums are stored slice-major: the value of column c of
// retained block rb sits at ((c / kFinCols) * n_part + rb) * kFinCols +
// c % kFinCols, so the rows k_pop_finish reads for one column slice are one
// contiguous run of n_part * kFinCols floats.
constexpr int kFinCols = POP_FIN_COLS;
#ifndef POP_FUSED_THREADS
#define POP_FUSED_THREADS 512  // threads of a k_pop_step / k_pop_linked block
#endif
constexpr int kFusedThreads = POP_FUSED_THREADS;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedTopkMaxN = 4096;
constexpr int kFusedMaxRows = 512;  // rows per block
#ifndef POP_FUSED_P
#define POP_FUSED_P 1
#endif
constexpr int kFusedP = POP_FUSED_P;  // rows per batch

template <typename T, int NV>
struct FusedRowBuf {
  u32x4 g[kFusedP][NV];
  u32x4 u[kFusedP][NV];
  u32x4 w[kFusedP][NV];
};

template <typename T, int NV, bool kDown>
__device__ __forceinline__ void fused_issue(FusedRowBuf<T, NV>& b, const int* rows, int i0, int nrows,
                                            const T* __restrict__ Wg, const T* __restrict__ Wu,
                                            const T* __restrict__ WdT, int d) {
  constexpr int V = Vec<T>::N;
  // No load carries a condition, so that the compiler's wait counting stays
  // exact across the double buffer (behind a branch, the count of the path
  // that skips a row applies to every path, and the consumer of one buffer
  // then waits for most of the other's loads too).  Lanes past the row's end
  // load its last vector, and slots past nrows load the list's last row again
  // (lines already requested by this block; their z is 0).  The scheduling
  // barriers keep the other buffer's arithmetic from being moved above these
  // loads, which would make it wait before they are issued.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < kFusedP; ++p) {
    const int64_t base = (int64_t)rows[min(i0 + p, nrows - 1)] * d;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int col = min(j * kFusedThreads * V + (int)threadIdx.x * V, d - V);
      b.g[p][j] = ld16_stream(Wg + base + col);
      b.u[p][j] = ld16_stream(Wu + base + col);
      if (kDown) b.w[p][j] = ld16_stream(WdT + base + col);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Reduces the batch's dot products across the block and applies them.
// Returns through zs the batch's z values (0 for rows past nrows).  No lane or
// row condition guards the arithmetic: columns past d hold x = 0, rows past
// nrows get z = 0, and every buffer slot holds a loaded (finite) weight.
template <typename T, int NV, bool kDown, int PB>
__device__ __forceinline__ void fused_consume(const FusedRowBuf<T, NV>& b, const u32x4 (&xv)[NV], int i0, int nrows,
                                              int d, float (&part)[2][kFusedWaves][2 * kFusedP], float (&acc)[NV][Vec<T>::N],
                                              float (&zs)[kFusedP]) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float pg[kFusedP], pu[kFusedP];
#pragma unroll
  for (int p = 0; p < kFusedP; ++p) {
    pg[p] = 0.f;
    pu[p] = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float g[V], u[V], xx[V];
      unpack(b.g[p][j], g, T{});
      unpack(b.u[p][j], u, T{});
      unpack(xv[j], xx, T{});
#pragma unroll
      for (int v = 0; v < V; ++v) {
        pg[p] = fmaf(g[v], xx[v], pg[p]);
        pu[p] = fmaf(u[v], xx[v], pu[p]);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kFusedP; ++p) {
    pg[p] = wave_sum_last(pg[p]);
    pu[p] = wave_sum_last(pu[p]);
  }
  if (lane == 63) {
#pragma unroll
    for (int p = 0; p < kFusedP; ++p) {
      part[PB][wave][2 * p] = pg[p];
      part[PB][wave][2 * p + 1] = pu[p];
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kFusedP; ++p) {
    float g = part[PB][0][2 * p], u = part[PB][0][2 * p + 1];
#pragma unroll
    for (int w = 1; w < kFusedWaves; ++w) {
      g += part[PB][w][2 * p];
      u += part[PB][w][2 * p + 1];
    }
    zs[p] = i0 + p < nrows ? silu(g) * u : 0.f;
  }
  if (kDown) {
#pragma unroll
    for (int p = 0; p < kFusedP; ++p) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float f[V];
        unpack(b.w[p][j], f, T{});
#pragma unroll
        for (int v = 0; v < V; ++v) acc[j][v] = fmaf(zs[p], f[v], acc[j][v]);
      }
    }
    // The products are due here: left to the optimiser they sink past the
    // next batch's loads, which then cannot reuse this buffer's registers
    // (the loop then copies a buffer at its back edge, waiting on its loads).
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int v = 0; v < V; ++v) asm volatile("" : "+v"(acc[j][v]));
  }
}

// Row i's z into zl[i] (LDS; thread 0), for the rows of the pair that exist.
__device__ __forceinline__ void fused_put_z(float* zl, int i0, int nrows, const float (&zs)[kFusedP]) {
  if (threadIdx.x == 0) {
#pragma unroll
    for (int p = 0; p < kFusedP; ++p)
      if (i0 + p < nrows) zl[i0 + p] = zs[p];
  }
}

// The rows rows[0 .. nrows) two at a time, double-buffered: the next pair's
// loads are issued before the current pair is reduced.  Every path issues
// the same loads (the last pairs are unrolled out of the loop rather than
// guarded), so each reduction waits only for its own pair.  z of row i goes
// to zl[i] (LDS, written by thread 0; the caller stores it after a barrier):
// a global store inside the loop would add to the counter the loads are
// waited on by.
template <typename T, int NV, bool kDown>
__device__ __forceinline__ void fused_rows(const int* rows, int nrows, const T* __restrict__ Wg, const T* __restrict__ Wu,
                                           const T* __restrict__ WdT, int d, const u32x4 (&xv)[NV],
                                           float (&part)[2][kFusedWaves][2 * kFusedP], float (&acc)[NV][Vec<T>::N],
                                           float* zl) {
  if (nrows <= 0) return;  // block-uniform
  FusedRowBuf<T, NV> A, Bf;
  float zs[kFusedP];
  fused_issue<T, NV, kDown>(A, rows, 0, nrows, Wg, Wu, WdT, d);
  int i0 = 0;
  for (; i0 + 2 * kFusedP < nrows; i0 += 2 * kFusedP) {
    fused_issue<T, NV, kDown>(Bf, rows, i0 + kFusedP, nrows, Wg, Wu, WdT, d);
    fused_consume<T, NV, kDown, 0>(A, xv, i0, nrows, d, part, acc, zs);
    fused_put_z(zl, i0, nrows, zs);
    fused_issue<T, NV, kDown>(A, rows, i0 + 2 * kFusedP, nrows, Wg, Wu, WdT, d);
    fused_consume<T, NV, kDown, 1>(Bf, xv, i0 + kFusedP, nrows, d, part, acc, zs);
    fused_put_z(zl, i0 + kFusedP, nrows, zs);
  }
  if (i0 + kFusedP < nrows) {  // two pairs left (the second possibly partial)
    fused_issue<T, NV, kDown>(Bf, rows, i0 + kFusedP, nrows, Wg, Wu, WdT, d);
    fused_consume<T, NV, kDown, 0>(A, xv, i0, nrows, d, part, acc, zs);
    fused_put_z(zl, i0, nrows, zs);
    fused_consume<T, NV, kDown, 1>(Bf, xv, i0 + kFusedP, nrows, d, part, acc, zs);
    fused_put_z(zl, i0 + kFusedP, nrows, zs);
  } else {  // one pair left
    fused_consume<T, NV, kDown, 0>(A, xv, i0, nrows, d, part, acc, zs);
    fused_put_z(zl, i0, nrows, zs);
  }
}

// Up to NB candidate rows at once (gate and up rows only): every load issued
// before any is used, so the batch costs one memory round trip, then one
// cross-wave reduction for all its rows.  Split into the issue and the
// reduction so that a caller can put other loads in flight in between.
template <typename T, int NV, int NB>
struct CandBuf {
  u32x4 g[NB][NV];
  u32x4 u[NB][NV];
};

template <typename T, int NV, int NB>
__device__ __forceinline__ void cand_issue(CandBuf<T, NV, NB>& b, const int* rows, int nrows,
                                           const T* __restrict__ Wg, const T* __restrict__ Wu, int d) {
  constexpr int V = Vec<T>::N;
#pragma unroll
  for (int p = 0; p < NB; ++p) {
    const int64_t base = (int64_t)rows[min(p, nrows - 1)] * d;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int col = min(j * kFusedThreads * V + (int)threadIdx.x * V, d - V);
      b.g[p][j] = ld16_stream(Wg + base + col);
      b.u[p][j] = ld16_stream(Wu + base + col);
    }
  }
}

// Threads p < nrows write row p's z to zout and zl (LDS, when not null), |z|
// to score and, when pub is set, its hand-over word pack_valid(bits of h,
// bits of z), with h = |z|, or with hm (an activation memory, copied to LDS)
// h = hm[p] + |z| while mclear[p] (the memory itself) is cleared.
template <typename T, int NV, int NB>
__device__ __forceinline__ void cand_consume(const CandBuf<T, NV, NB>& b, int nrows, const u32x4 (&xv)[NV],
                                             float (&part)[kFusedWaves][2 * NB], float* __restrict__ zout,
                                             float* __restrict__ score, uint64_t* __restrict__ pub, float* zl,
                                             const float* hm = nullptr, float* __restrict__ mclear = nullptr) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float pg[NB], pu[NB];
#pragma unroll
  for (int p = 0; p < NB; ++p) {
    pg[p] = pu[p] = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float gf[V], uf[V], xx[V];
      unpack(b.g[p][j], gf, T{});
      unpack(b.u[p][j], uf, T{});
      unpack(xv[j], xx, T{});
#pragma unroll
      for (int v = 0; v < V; ++v) {
        pg[p] = fmaf(gf[v], xx[v], pg[p]);
        pu[p] = fmaf(uf[v], xx[v], pu[p]);
      }
    }
    pg[p] = wave_sum_last(pg[p]);
    pu[p] = wave_sum_last(pu[p]);
  }
  if (lane == 63) {
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      part[wave][2 * p] = pg[p];
      part[wave][2 * p + 1] = pu[p];
    }
  }
  __syncthreads();
  if (threadIdx.x < NB && (int)threadIdx.x < nrows) {
    const int p = threadIdx.x;
    float gs = part[0][2 * p], us = part[0][2 * p + 1];
#pragma unroll
    for (int w = 1; w < kFusedWaves; ++w) {
      gs += part[w][2 * p];
      us += part[w][2 * p + 1];
    }
    const float zz = silu(gs) * us;
    zout[p] = zz;
    score[p] = fabsf(zz);
    if (zl != nullptr) zl[p] = zz;
    if (pub != nullptr) {
      const float h = hm != nullptr ? hm[p] + fabsf(zz) : fabsf(zz);
      st_coh(&pub[p], pack_valid(__float_as_uint(h), __float_as_uint(zz)));
    }
    if (mclear != nullptr) mclear[p] = 0.f;
  }
  __syncthreads();  // part is reused by the next batch
}

// Loads this thread's x vectors and clears its down accumulators.
template <typename T, int NV>
__device__ __forceinline__ void fused_setup(const T* __restrict__ x, int d, u32x4 (&xv)[NV],
                                            float (&acc)[NV][Vec<T>::N]) {
  constexpr int V = Vec<T>::N;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int col = j * kFusedThreads * V + (int)threadIdx.x * V;
    xv[j] = col < d ? ld16(x + col) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int v = 0; v < V; ++v) acc[j][v] = 0.f;
  }
}

// Launch-invariant arguments of k_pop_step, kept as separate restrict-qualified
// kernel parameters (a by-value struct loses the no-alias information and the
// retained stream measured about 8% slower that way).
#define POP_STEP_PARAMS                                                                                          \
  const T *__restrict__ x, const T *__restrict__ Wg, const T *__restrict__ Wu, const T *__restrict__ WdT,        \
      const int32_t *__restrict__ R, const int32_t *__restrict__ C, float *__restrict__ z,                       \
      float *__restrict__ score, int32_t *__restrict__ Q, int32_t *__restrict__ sel, float *__restrict__ partial, \
      int d, int d_ff, int n_R, int n_C, int k, int rows_per_cblock, int rows_per_rblock, int nb0, int rb_base,  \
      int n_part

struct NoSel {};

// One launch of the batch-1 step.  Blocks [0, nb0) run the phase's link of the
// candidate chain (see above; PHASE 0 has no chain link: every block is a
// retained block, compiled without the chain's code); block nb0 + b runs
// retained block rb_base + b: rows R[rb * rows_per_rblock, ...) (rows
// rb * rows_per_rblock, ... with kIdentity), their z, and its partial
// y = sum of z * W_downT[ch, :].
template <typename T, int NV, bool kIdentity, int PHASE>
__global__ __launch_bounds__(kFusedThreads) void k_pop_step(POP_STEP_PARAMS) {
  static_assert(PHASE >= 0 && PHASE <= 2, "phases 0, 1, 2");
  constexpr int V = Vec<T>::N;
  using SelT = typename std::conditional<PHASE == 2, SelShared<kFusedThreads, kFusedTopkMaxN>, NoSel>::type;
  __shared__ SelT sh_sel;
  __shared__ int rows[kFusedMaxRows];
  __shared__ float zl[kFusedMaxRows];
  __shared__ float part[2][kFusedWaves][2 * kFusedP];
  const int bid = blockIdx.x;
  if (PHASE != 0 && bid < nb0) {
    if constexpr (PHASE == 0) {
    } else if constexpr (PHASE == 1) {  // candidate rows: z (after the n_R retained entries) and scores |z|
      u32x4 xv[NV];
      float acc[NV][V];
      fused_setup<T, NV>(x, d, xv, acc);
      const int r0 = bid * rows_per_cblock;
      const int nrows = max(0, min(n_C, r0 + rows_per_cblock) - r0);
      for (int i = threadIdx.x; i < nrows; i += kFusedThreads) rows[i] = clamp_channel(C[r0 + i], d_ff);
      __syncthreads();
      fused_rows<T, NV, false>(rows, nrows, Wg, Wu, (const T*)nullptr, d, xv, part, acc, zl);
      __syncthreads();
      for (int i = threadIdx.x; i < nrows; i += kFusedThreads) {
        z[n_R + r0 + i] = zl[i];
        score[r0 + i] = fabsf(zl[i]);
      }
    } else {  // the top-k over the scores phase 1 wrote
      topk_block(score, n_C, k, C, Q, sel, sh_sel);
    }
    return;
  }
  u32x4 xv[NV];
  float acc[NV][V];
  fused_setup<T, NV>(x, d, xv, acc);
  const int rb = rb_base + bid - nb0;
  const int r0 = rb * rows_per_rblock;
  const int nrows = max(0, min(n_R, r0 + rows_per_rblock) - r0);
  for (int i = threadIdx.x; i < nrows; i += kFusedThreads) rows[i] = kIdentity ? r0 + i : clamp_channel(R[r0 + i], d_ff);
  __syncthreads();
  fused_rows<T, NV, true>(rows, nrows, Wg, Wu, WdT, d, xv, part, acc, zl);
  __syncthreads();
  for (int i = threadIdx.x; i < nrows; i += kFusedThreads) z[r0 + i] = zl[i];
  static_assert(kFinCols % V == 0, "a thread's columns lie in one slice");
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int col = j * kFusedThreads * V + (int)threadIdx.x * V;
    if (col < d) {
      float* out = partial + ((int64_t)(col / kFinCols) * n_part + rb) * kFinCols + col % kFinCols;
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = acc[j][v];
    }
  }
}
#undef POP_STEP_PARAMS

// The last launch of the batch-1 step.  Block s owns the kFinCols columns
// c0 = s * kFinCols + [0, kFinCols) of y and adds, in a fixed order, the
// n_part retained partial sums and (kSel) the k selected rows' z * W_downT,
// then writes y itself (no partial of its own).  512 threads = 8 waves:
//   partial rows (slice-major, contiguous): kFinCols / 4 lanes x 4 floats per row;
//   selected rows: kFinCols / V lanes x 16 bytes per row; row j of S is
//   (ch, z) = (sel[j], z[zoff + pos[j]]).
// Issue order: the first batch's selected-row indices, the first batch of
// partial rows, then (once the indices are in) the selected rows' z and
// W_downT, and only then the partial sums are consumed: for up to
// kFinRowsPerBatch selected rows and kFinPB * PPB partials every load is in
// flight at once.  The per-lane sums are reduced across lanes (shuffles), then
// across waves in wave order (LDS).
#ifndef POP_FIN_THREADS
#define POP_FIN_THREADS 512
#endif
constexpr int kFinThreads = POP_FIN_THREADS;
// Control word of the single-launch batch-1 step: the sticky error word.
constexpr int kCtlErr = 0;
constexpr int kFinRowsPerBatch = 1280;  // selected rows whose loads are in flight together
constexpr int kFinPartials = 512;       // partial rows whose loads are in flight together

// Block b's column slice.  With slices narrower than 64 columns, the slices
// of one 128-byte bf16 W_downT line go to blocks on the same XCD (blocks are
// dealt to the eight XCDs round-robin), so the line is fetched into one L2.
__device__ __forceinline__ int fin_slice(int b, int nb) {
  constexpr int SP = kFinCols >= 64 ? 1 : 64 / kFinCols;  // slices per line
  constexpr int G = 8 * SP;                                // blocks per group
  if (SP == 1 || (b | (G - 1)) >= nb) return b;            // the last, partial group keeps its order
  const int q = b / G, h = (b / 8) % SP, x = b % 8;
  return (q * 8 + x) * SP + h;
}

// The periodic mode's memory update of a kept step, done by the step's last
// launch: mem[pos[j]] += |z[zoff + j]| for j < k (batch 1; mem NULL: none).
struct MemAdd {
  float* mem;
  const int32_t* pos;
  int zoff, k, n_C;
};

template <typename T, bool kSel, bool kMem = false>
__global__ __launch_bounds__(kFinThreads) void k_pop_finish(const float* __restrict__ partial, int n_part,
                                                            const float* __restrict__ z, int zoff, int n_A,
                                                            const int32_t* __restrict__ sel,
                                                            const int32_t* __restrict__ pos, int k,
                                                            const T* __restrict__ WdT, int d, int d_ff,
                                                            float* __restrict__ y, int accumulate,
                                                            uint64_t* reset_words, int n_reset_words,
                                                            MemAdd ma) {
  constexpr int V = Vec<T>::N;
  constexpr int LR = kFinCols / V;       // lanes per W_downT row
  constexpr int RPW = 64 / LR;           // W_downT rows per wave instruction
  constexpr int RPB = RPW * (kFinThreads / 64);
  constexpr int LP = kFinCols / 4;       // lanes per partial row
  constexpr int PPW = 64 / LP;           // partial rows per wave instruction
  constexpr int PPB = PPW * (kFinThreads / 64);
  constexpr int PB = (kFinPartials + PPB - 1) / PPB;           // partial-row loads in flight per lane
  constexpr int SB = (kFinRowsPerBatch + RPB - 1) / RPB;       // selected-row loads in flight per lane
  __shared__ float red[kFinThreads / 64][kFinCols];
  // the single-launch step's hand-over words, cleared for the next call
  for (int i = blockIdx.x * kFinThreads + threadIdx.x; i < n_reset_words; i += gridDim.x * kFinThreads)
    st_coh(&reset_words[i], (uint64_t)0);
  if constexpr (kMem)  // positions are distinct: one thread per entry
    for (int j = blockIdx.x * kFinThreads + threadIdx.x; j < ma.k; j += gridDim.x * kFinThreads) {
      const int p = ma.pos[j];
      if (p >= 0 && p < ma.n_C) ma.mem[p] += fabsf(z[ma.zoff + j]);
    }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = fin_slice(blockIdx.x, gridDim.x) * kFinCols;
  const int jl = wave * RPW + lane / LR;  // this lane's selected row within a block instruction
  const int pl = wave * PPW + lane / LP;  // this lane's partial row within a block instruction
  const float* pslice = partial + (int64_t)(c0 / kFinCols) * n_part * kFinCols + (lane % LP) * 4;
  const int colw = min(c0 + (lane % LR) * V, d - V);
  float ap[4] = {0.f, 0.f, 0.f, 0.f};
  float as[V];
#pragma unroll
  for (int v = 0; v < V; ++v) as[v] = 0.f;
  // raw indices; clamped where they are used, so nothing waits on them early
  int ch[SB], zi[SB];
  float zv[SB];
  u32x4 w[SB];
  float4 pv[PB];
  auto load_idx = [&](int j0) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int j = max(0, min(j0 + u * RPB + jl, k - 1));
      ch[u] = sel[j];
      zi[u] = pos[j];
    }
  };
  auto issue_sel = [&]() {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      zv[u] = z[min(zoff + max(zi[u], 0), n_A - 1)];
      w[u] = ld16_stream(WdT + (int64_t)clamp_channel(ch[u], d_ff) * d + colw);
    }
  };
  auto consume_sel = [&](int j0) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float zz = j0 + u * RPB + jl < k ? zv[u] : 0.f;
      float f[V];
      unpack(w[u], f, T{});
#pragma unroll
      for (int v = 0; v < V; ++v) as[v] = fmaf(zz, f[v], as[v]);
    }
  };
  auto issue_part = [&](int p0) {
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int p = max(0, min(p0 + u * PPB + pl, n_part - 1));
      pv[u] = *reinterpret_cast<const float4*>(pslice + (int64_t)p * kFinCols);
    }
  };
  auto consume_part = [&](int p0) {
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      // a select, not a product: rows past n_part may hold anything
      const bool on = p0 + u * PPB + pl < n_part;
      ap[0] += on ? pv[u].x : 0.f;
      ap[1] += on ? pv[u].y : 0.f;
      ap[2] += on ? pv[u].z : 0.f;
      ap[3] += on ? pv[u].w : 0.f;
    }
  };
  // first batches: every load in flight before any is consumed (sel, pos and
  // partial hold at least one entry, so the loads carry no condition)
  if constexpr (kSel) load_idx(0);
  issue_part(0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kSel) issue_sel();
  __builtin_amdgcn_sched_barrier(0);
  consume_part(0);
  for (int p0 = PB * PPB; p0 < n_part; p0 += PB * PPB) {
    issue_part(p0);
    consume_part(p0);
  }
  if constexpr (kSel) {
    consume_sel(0);
    for (int j0 = SB * RPB; j0 < k; j0 += SB * RPB) {
      load_idx(j0);
      issue_sel();
      consume_sel(j0);
    }
  }
  // ---- lanes with the same columns: fixed butterfly order
#pragma unroll
  for (int o = LP; o < 64; o <<= 1)
#pragma unroll
    for (int v = 0; v < 4; ++v) ap[v] += __shfl_xor(ap[v], o);
#pragma unroll
  for (int o = LR; o < 64; o <<= 1)
#pragma unroll
    for (int v = 0; v < V; ++v) as[v] += __shfl_xor(as[v], o);
  // lanes 0..LP-1 hold the partials' sums of columns 4 * lane + [0, 4);
  // lanes 0..LR-1 hold the selected rows' sums of columns V * lane + [0, V)
  if (lane < LP) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][lane * 4 + v] = ap[v];
  }
  __syncthreads();
  if (lane < LR) {
#pragma unroll
    for (int v = 0; v < V; ++v) red[wave][lane * V + v] += as[v];
  }
  __syncthreads();
  if (threadIdx.x < kFinCols && c0 + (int)threadIdx.x < d) {
    float t = red[0][threadIdx.x];
#pragma unroll
    for (int w2 = 1; w2 < kFinThreads / 64; ++w2) t += red[w2][threadIdx.x];
    y[c0 + threadIdx.x] = accumulate ? y[c0 + threadIdx.x] + t : t;  // accumulate: y += FFN(x)
  }
}

// ---------------------------------------------------------------- single-launch batch-1 step
// The batch-1 step in two launches, the candidate chain running inside the
// retained stream of the first.  Block 0 of k_pop_linked is the candidate
// top-k; blocks 1 .. nW are workers, and worker w takes an even share
// (split_at) of each list:
//   1. its candidate rows: gate and up rows, z (kept in LDS) and |z|; each
//      row's (|z|, z) goes to block 0 as one valid-tagged word.  The loads of
//      its first retained rows are issued before the last candidate batch is
//      reduced;
//   2. its retained rows: gate, up and W_downT rows, z, and z * W_downT added
//      into its partial y (registers); every second row batch also re-reads
//      the published cut (one coherent 8-byte load beside the rows' loads);
//   3. the selected rows: block 0 publishes the cut (v, tie position), then
//      writes the selected candidates, in position order, as valid-tagged
//      (channel, z) pairs.  Worker w adds the selected rows of ranks
//      split_at(k, nW, w) .. split_at(k, nW, w + 1), an equal share whoever
//      owned the candidates.  Wave 0 looks at the cut it read two batch pairs
//      earlier; once it is out, it loads the worker's pairs (coherent), and
//      two pairs later, if all are valid, puts them in LDS and flags them
//      ready (else it loads them again).  If they are ready before the last
//      two row batches, their W_downT rows' loads go out with those batches;
//      otherwise the worker polls for its pairs after its rows and adds the
//      rows then.  Both ways add the same rows in the same order;
//   4. its partial y, slice-major, with plain stores.
// k_pop_finish then adds the nW partials in a fixed order into y and clears
// the hand-over words for the next call.  Only block 0 waits on many
// workgroups (one poller); a worker waits at most for the cut.  Nothing
// waits on a workgroup that is not running: the host keeps the grid within
// what the device holds at once, and block 0 needs only the workers' first
// phase.  Every wait is bounded (kPollLimit polls); one that runs out sets
// the sticky error word ctl[kCtlErr] and the step goes on (its y is then
// wrong).
#ifndef POP_LINKED_ON
#define POP_LINKED_ON 1  // 0: batch-1 steps take the three-launch path
#endif
constexpr int kLinkedTopkMaxN = 4096;
constexpr int kLinkedMaxWorkers = POP_FUSED_RBLOCKS - 1;
constexpr int kPollLimit = 1 << 20;
#ifndef POP_LINKED_NS
#define POP_LINKED_NS 8
#endif
constexpr int kLinkedNS = POP_LINKED_NS;  // selected rows carried by the last row batches (and per later pass)
constexpr int kThrCopies = 32;  // copies of the published cut
constexpr int kThrStride = 16;  // 64-bit words between copies (128 bytes)
#ifndef POP_CAND_BATCH
#define POP_CAND_BATCH 3
#endif
constexpr int kCandBatch = POP_CAND_BATCH;  // candidate rows whose loads a worker issues together
// The control words (1 KB), then the hand-over words: the candidate words (at
// most kLinkedTopkMaxN), the copies of the cut, and the selected pairs (at
// most kLinkedTopkMaxN).  A fixed region at the start of every decode
// workspace that no other call writes; k_pop_finish leaves it zero (the error
// word aside).
constexpr size_t kCtlBytes = 1024;
constexpr size_t kPairsWord = kLinkedTopkMaxN + kThrCopies * kThrStride;  // first pair word
constexpr size_t kHandWords = kPairsWord + kLinkedTopkMaxN;
constexpr size_t kHandBytes = kHandWords * sizeof(uint64_t);
static_assert(kHandBytes % 256 == 0, "z stays 256-byte aligned");

__device__ __forceinline__ int split_at(int n, int parts, int i) { return (int)(((int64_t)n * i) / parts); }

// The W_downT rows of up to NS selected candidates, every load issued at
// once; slots past n load the list's last row again (n >= 1).
template <typename T, int NV, int NS>
__device__ __forceinline__ void sel_issue(u32x4 (&ws)[NS][NV], const int* chan, int n, const T* __restrict__ WdT,
                                          int d, int d_ff) {
  constexpr int V = Vec<T>::N;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    const int64_t base = (int64_t)clamp_channel(chan[min(q, n - 1)], d_ff) * d;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int col = min(j * kFusedThreads * V + (int)threadIdx.x * V, d - V);
      ws[q][j] = ld16_stream(WdT + base + col);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Adds z_q * W_downT[chan_q, :] for q < n, in order (slots past n add
// nothing: they are skipped, not multiplied by zero).
template <typename T, int NV, int NS>
__device__ __forceinline__ void sel_consume(const u32x4 (&ws)[NS][NV], const float* zv, int n,
                                            float (&acc)[NV][Vec<T>::N]) {
  constexpr int V = Vec<T>::N;
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    if (q < n) {  // block-uniform
      const float zz = zv[q];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float f[V];
        unpack(ws[q][j], f, T{});
#pragma unroll
        for (int v = 0; v < V; ++v) acc[j][v] = fmaf(zz, f[v], acc[j][v]);
      }
    }
  }
}

// The last one or two row batches of a worker's stream (X holds batch i0, its
// loads in flight; PB0 is the partial-sum buffer of the first reduction
// here), and the worker's share of the selected rows (m of them) when wave 0
// has them in s_chan / s_zv already (*sh_ready): the first NS are added after
// the rows, their loads issued with the last batches.  Returns how many were
// added, or -1 when the share was not ready in time.
template <typename T, int NV, int NS, int PB0>
__device__ __forceinline__ int linked_last(FusedRowBuf<T, NV>& X, FusedRowBuf<T, NV>& Y, int i0, const int* rows,
                                           int nrows, const T* __restrict__ Wg, const T* __restrict__ Wu,
                                           const T* __restrict__ WdT, int d, int d_ff, const u32x4 (&xv)[NV],
                                           float (&part)[2][kFusedWaves][2 * kFusedP],
                                           float (&acc)[NV][Vec<T>::N], float* zl, bool sel_here, int m,
                                           const int* s_chan, const float* s_zv, const int* sh_ready, int* sh_nsel) {
  const int nl = max(nrows, 1);
  float zs[kFusedP];
  // Wave 0 (thread 0's wave) wrote the share and the ready flag; the block
  // takes the decision from LDS.
  if (threadIdx.x == 0) *sh_nsel = sel_here && *sh_ready != 0 ? m : -1;
  lds_barrier();
  const int got = *sh_nsel;  // block-uniform; -1: the share was not ready
  const bool early = got >= 0;
  const int nsl = early ? min(got, NS) : 0;
  u32x4 ws[NS][NV];
  const int* srow = nsl > 0 ? s_chan : rows + (nl - 1);
  if (i0 + kFusedP < nrows) {  // two batches left
    fused_issue<T, NV, true>(Y, rows, i0 + kFusedP, nl, Wg, Wu, WdT, d);
    sel_issue<T, NV, NS>(ws, srow, max(nsl, 1), WdT, d, d_ff);
    fused_consume<T, NV, true, PB0>(X, xv, i0, nrows, d, part, acc, zs);
    fused_put_z(zl, i0, nrows, zs);
    fused_consume<T, NV, true, 1 - PB0>(Y, xv, i0 + kFusedP, nrows, d, part, acc, zs);
    fused_put_z(zl, i0 + kFusedP, nrows, zs);
  } else {
    sel_issue<T, NV, NS>(ws, srow, max(nsl, 1), WdT, d, d_ff);
    fused_consume<T, NV, true, PB0>(X, xv, i0, nrows, d, part, acc, zs);
    fused_put_z(zl, i0, nrows, zs);
  }
  sel_consume<T, NV, NS>(ws, s_zv, nsl, acc);
  return early ? nsl : -1;
}

// A worker's retained rows rows[0 .. nrows), double-buffered (the first
// batch's loads already issued into A by the caller; rows holds at least one
// entry even when nrows is 0, whose loads then go unused), the cut re-read
// beside every second batch, and the ending of linked_last.  The first batch
// is reduced before the loop, so the buffer the loop carries is issued right
// before it.  Wave 0 also fetches the worker's share of the selected pairs
// (pairs[s0 .. s0 + m), at most 64) once the cut it read two iterations
// earlier is out; each step uses only values loaded an iteration or more
// before, so no wait is added to the stream, and a pair not yet valid is
// loaded again.
template <typename T, int NV, int NS>
__device__ __forceinline__ int linked_stream(FusedRowBuf<T, NV>& A, const int* rows, int nrows,
                                             const T* __restrict__ Wg, const T* __restrict__ Wu,
                                             const T* __restrict__ WdT, int d, int d_ff, const u32x4 (&xv)[NV],
                                             float (&part)[2][kFusedWaves][2 * kFusedP],
                                             float (&acc)[NV][Vec<T>::N], float* zl, bool sel_here,
                                             const uint64_t* cutw, const uint64_t* pairs, int s0, int m,
                                             int* s_chan, float* s_zv, int* sh_ready, int* sh_nsel) {
  const int nl = max(nrows, 1);
  FusedRowBuf<T, NV> Bf, A2;
  float zs[kFusedP];
  if (nrows <= 2 * kFusedP)
    return linked_last<T, NV, NS, 0>(A, Bf, 0, rows, nrows, Wg, Wu, WdT, d, d_ff, xv, part, acc, zl, sel_here, m,
                                     s_chan, s_zv, sh_ready, sh_nsel);
  const int lane = threadIdx.x & 63;
  const bool fetcher = sel_here && m <= 64 && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;  // wave-uniform
  uint64_t cw = ld_coh(cutw), cw_old = 0, pv = 0;
  int st = fetcher ? 0 : 3;  // 0: cut not seen; 1, 2: pairs in flight; 3: done (or not this wave's job)
  fused_issue<T, NV, true>(Bf, rows, kFusedP, nl, Wg, Wu, WdT, d);
  fused_consume<T, NV, true, 0>(A, xv, 0, nrows, d, part, acc, zs);
  fused_put_z(zl, 0, nrows, zs);
  int i0 = kFusedP;  // Bf holds batch i0
  for (; i0 + 2 * kFusedP < nrows; i0 += 2 * kFusedP) {
    if (st < 3) {  // wave-uniform: wave 0 only
      if (st == 0) {
        if (is_valid(cw_old)) {  // read two iterations ago: complete
          pv = ld_coh(&pairs[s0 + min(lane, m - 1)]);
          st = 1;
        }
      } else if (st == 1) {
        st = 2;
      } else if (__ballot(lane < m && !is_valid(pv)) != 0) {  // loaded two iterations ago; not all in yet
        pv = ld_coh(&pairs[s0 + min(lane, m - 1)]);
        st = 1;
      } else {
        if (lane < m) {
          s_chan[lane] = clamp_channel((int)((uint32_t)(pv >> 32) & 0x7fffffffu), d_ff);
          s_zv[lane] = __uint_as_float((uint32_t)pv);
        }
        if (lane == 0) *sh_ready = 1;  // after the share: one wave's LDS stores stay in order
        st = 3;
      }
    }
    cw_old = cw;
    fused_issue<T, NV, true>(A2, rows, i0 + kFusedP, nl, Wg, Wu, WdT, d);
    cw = ld_coh(cutw);
    fused_consume<T, NV, true, 1>(Bf, xv, i0, nrows, d, part, acc, zs);
    fused_put_z(zl, i0, nrows, zs);
    fused_issue<T, NV, true>(Bf, rows, i0 + 2 * kFusedP, nl, Wg, Wu, WdT, d);
    fused_consume<T, NV, true, 0>(A2, xv, i0 + kFusedP, nrows, d, part, acc, zs);
    fused_put_z(zl, i0 + kFusedP, nrows, zs);
  }
  return linked_last<T, NV, NS, 1>(Bf, A2, i0, rows, nrows, Wg, Wu, WdT, d, d_ff, xv, part, acc, zl, sel_here, m,
                                   s_chan, s_zv, sh_ready, sh_nsel);
}

#ifndef POP_LINKED_MINB
#define POP_LINKED_MINB 1  // workgroups of k_pop_linked resident per CU
#endif
template <typename T, int NV, bool kIdentity, bool kMem>
__global__ __launch_bounds__(kFusedThreads, POP_LINKED_MINB) void k_pop_linked(
    const T* __restrict__ x, const T* __restrict__ Wg, const T* __restrict__ Wu, const T* __restrict__ WdT,
    const int32_t* __restrict__ R, const int32_t* __restrict__ C, float* __restrict__ z, float* __restrict__ score,
    uint64_t* __restrict__ hand, int32_t* __restrict__ sel_out, float* __restrict__ partial,
    uint32_t* __restrict__ ctl, uint64_t* __restrict__ pairs, int d, int d_ff, int n_R, int n_C, int k, int nW,
    float* __restrict__ mem, int32_t* __restrict__ pos_out) {
  constexpr int V = Vec<T>::N;
  struct Work {
    int rows[kFusedMaxRows];
    float zr[kFusedMaxRows];  // z of this worker's retained rows
    float cm[kFusedMaxRows];  // the activation memory of this worker's candidates (periodic refresh)
    float part[2][kFusedWaves][2 * kFusedP];
    float cpart[kFusedWaves][2 * kCandBatch];
    int crow[kFusedMaxRows];  // this worker's share of C (channels)
    int n_sel;
    int ready;                  // s_chan / s_zv hold the share (set by wave 0)
    int s_chan[kFusedMaxRows];  // this worker's share of the selected candidates: channel and z
    float s_zv[kFusedMaxRows];
  };
  __shared__ union {
    SelShared<kFusedThreads, kLinkedTopkMaxN> sel;
    Work w;
  } sh;
  const int tid = threadIdx.x;
  const bool chain = n_C > 0 && k > 0;  // a top-k runs
  uint64_t* cand = hand;
  uint64_t* thr = hand + kLinkedTopkMaxN;
  if (blockIdx.x == 0) {
    if (chain)
      topk_threshold_linked(cand, n_C, k, C, pos_out, sel_out, thr, kThrCopies, kThrStride, sh.sel, kPollLimit,
                            ctl + kCtlErr, nullptr, pairs);
    return;
  }
  const int w = blockIdx.x - 1;
  const int c0 = split_at(n_C, nW, w), nc = split_at(n_C, nW, w + 1) - c0;
  const int r0 = split_at(n_R, nW, w), nr = split_at(n_R, nW, w + 1) - r0;
  const int s0 = split_at(k, nW, w), m = split_at(k, nW, w + 1) - s0;  // this worker's selected ranks
  u32x4 xv[NV];
  float acc[NV][V];
  fused_setup<T, NV>(x, d, xv, acc);
  for (int i = tid; i < nc; i += kFusedThreads) sh.w.crow[i] = clamp_channel(C[c0 + i], d_ff);
  if constexpr (kMem)
    for (int i = tid; i < nc; i += kFusedThreads) sh.w.cm[i] = mem[c0 + i];
  for (int i = tid; i < nr; i += kFusedThreads) sh.w.rows[i] = kIdentity ? r0 + i : clamp_channel(R[r0 + i], d_ff);
  if (tid == 0) sh.w.ready = 0;
  __syncthreads();
  const bool sel_here = chain && m > 0;
  const uint64_t* cutw = thr + (w % kThrCopies) * kThrStride;
  // with no retained rows, the stream's (unused) loads read the first candidate's rows
  const int* rlist = nr > 0 ? sh.w.rows : sh.w.crow;
  FusedRowBuf<T, NV> A;
  // 1. candidate rows, KB at a time, double-buffered: batch b + 1's loads go
  //    out before batch b is reduced, and the first retained rows' loads
  //    before the last batch is.  Every pass of the loop issues the same
  //    loads (no load behind a branch), so the compiler's wait counts stay
  //    exact; the one or two batches after it are straight-line code.
  constexpr int KB = kCandBatch / NV > 0 ? kCandBatch / NV : 1;
  auto cand_at = [&](CandBuf<T, NV, KB>& b, int q) {
    cand_issue<T, NV, KB>(b, sh.w.crow + q * KB, nc - q * KB, Wg, Wu, d);
  };
  auto cand_done = [&](const CandBuf<T, NV, KB>& b, int q) {
    const int i0 = q * KB;
    // the first KB pairs of columns of the LDS partials (KB <= kCandBatch)
    auto& cp = *reinterpret_cast<float(*)[kFusedWaves][2 * KB]>(&sh.w.cpart[0][0]);
    cand_consume<T, NV, KB>(b, min(KB, nc - i0), xv, cp, z + n_R + c0 + i0, score + c0 + i0,
                            chain ? cand + c0 + i0 : nullptr, nullptr, kMem ? sh.w.cm + i0 : nullptr,
                            kMem ? mem + c0 + i0 : nullptr);
  };
  if (nc > 0) {
    const int nb = (nc + KB - 1) / KB;
    CandBuf<T, NV, KB> ca, cb;
    cand_at(ca, 0);
    int b = 0;  // ca holds batch b
    for (; b + 2 < nb; b += 2) {
      cand_at(cb, b + 1);
      cand_done(ca, b);
      cand_at(ca, b + 2);
      cand_done(cb, b + 1);
    }
    if (b + 2 == nb) {
      cand_at(cb, b + 1);
      cand_done(ca, b);
      fused_issue<T, NV, true>(A, rlist, 0, max(nr, 1), Wg, Wu, WdT, d);
      cand_done(cb, b + 1);
    } else {
      fused_issue<T, NV, true>(A, rlist, 0, max(nr, 1), Wg, Wu, WdT, d);
      cand_done(ca, b);
    }
  } else {
    fused_issue<T, NV, true>(A, rlist, 0, max(nr, 1), Wg, Wu, WdT, d);
  }
  // 2. retained rows (and, when the cut is out in time, the selected rows)
  int done = linked_stream<T, NV, kLinkedNS>(A, rlist, nr, Wg, Wu, WdT, d, d_ff, xv, sh.w.part, acc, sh.w.zr, sel_here,
                                             cutw, pairs, s0, m, sh.w.s_chan, sh.w.s_zv, &sh.w.ready, &sh.w.n_sel);
  __syncthreads();
  for (int i = tid; i < nr; i += kFusedThreads) z[r0 + i] = sh.w.zr[i];
  // 3. otherwise this worker's share of the selected pairs now, each polled
  //    until valid (a wait that runs out leaves z = 0 and sets the error word)
  int ns = 0;
  if (sel_here) {
    if (done < 0) {
      for (int i = tid; i < m; i += kFusedThreads) {
        bool ok;
        const uint64_t pv = poll_coh(&pairs[s0 + i], [](uint64_t v) { return is_valid(v); }, kPollLimit, ok);
        if (!ok) st_coh(ctl + kCtlErr, 2u);
        sh.w.s_chan[i] = clamp_channel((int)((uint32_t)(pv >> 32) & 0x7fffffffu), d_ff);
        sh.w.s_zv[i] = ok ? __uint_as_float((uint32_t)pv) : 0.f;
      }
      __syncthreads();
      done = 0;
    }
    ns = m;
  }
  // done is -1 for a worker with no share (linked_last's "not early")
  for (int q0 = max(done, 0); q0 < ns; q0 += kLinkedNS) {
    u32x4 ws[kLinkedNS][NV];
    const int nq = min(kLinkedNS, ns - q0);
    sel_issue<T, NV, kLinkedNS>(ws, sh.w.s_chan + q0, nq, WdT, d, d_ff);
    sel_consume<T, NV, kLinkedNS>(ws, sh.w.s_zv + q0, nq, acc);
  }
  // 4. partial y, slice-major: column c of worker w at ((c / kFinCols) * nW + w) * kFinCols + c % kFinCols
  static_assert(kFinCols % V == 0, "a thread's columns lie in one slice");
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int col = j * kFusedThreads * V + tid * V;
    if (col < d) {
      float* out = partial + ((int64_t)(col / kFinCols) * nW + w) * kFinCols + col % kFinCols;
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = acc[j][v];
    }
  }
}

// ---------------------------------------------------------------- K6
// Block: 256 threads = 4 waves sharing one column slice of 64*V columns.  The
// block owns a chunk of live rows; wave w takes rows q0 + w, q0 + w + 4, ...
// Each wave first loads the channel and z column of up to 64 of its rows in one
// coalesced load (lane l holds row l), then streams the rows U at a time, each
// lane reading one 16-byte vector of every row (a wave reads 1 KB of a bf16
// row).  Live row q is (ch, zcol) = (R[q], q) for q < n_R and
// (sel[q - n_R], zoff + pos[q - n_R]) after; with kIdentity it is (q, q).
// The four wave accumulators are combined in wave order through LDS and written
// as this chunk's partial sum.
template <typename T, int BT, bool kIdentity>
__global__ __launch_bounds__(256) void k_down_partial(const float* __restrict__ z, int n_A, int B,
                                                      const T* __restrict__ WdT, int d, int d_ff,
                                                      const int32_t* __restrict__ R, int n_R,
                                                      const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ pos, int zoff, int n_live,
                                                      int rows_per_chunk, float* __restrict__ partial) {
  constexpr int V = Vec<T>::N;
  constexpr int U = BT == 1 ? 16 : 8;
  __shared__ float red[3][BT * V][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (blockIdx.x * 64 + lane) * V;
  const bool on = col < d;
  const int q0 = blockIdx.y * rows_per_chunk;
  const int q1 = min(n_live, q0 + rows_per_chunk);
  const int my_rows = q1 - q0 - wave > 0 ? (q1 - q0 - wave + 3) / 4 : 0;
  for (int b0 = 0; b0 < B; b0 += BT) {
    float acc[BT][V];
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int v = 0; v < V; ++v) acc[b][v] = 0.f;
    for (int r0 = 0; r0 < my_rows; r0 += 64) {
      // lane l: index of this wave's row r0 + l
      const int ql = q0 + wave + 4 * (r0 + lane);
      int ch_l = 0, zc_l = 0;
      if (r0 + lane < my_rows) {
        if (kIdentity) {
          ch_l = ql;
          zc_l = ql;
        } else if (ql < n_R) {
          ch_l = clamp_channel(R[ql], d_ff);
          zc_l = ql;
        } else {
          ch_l = clamp_channel(sel[ql - n_R], d_ff);
          zc_l = min(zoff + max(pos[ql - n_R], 0), n_A - 1);
        }
      }
      const int cnt = min(64, my_rows - r0);
      for (int j = 0; j < cnt; j += U) {
        u32x4 w[U];
        int zc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int src = j + u < 64 ? j + u : 63;  // lanes past cnt are never used
          const int ch = __builtin_amdgcn_readlane(ch_l, src);
          zc[u] = __builtin_amdgcn_readlane(zc_l, src);
          if (on && j + u < cnt) w[u] = ld16_stream(WdT + (int64_t)ch * d + col);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (on && j + u < cnt) {
            float f[V];
            unpack(w[u], f, T{});
#pragma unroll
            for (int b = 0; b < BT; ++b) {
              if (b0 + b < B) {
                const float zb = z[(int64_t)(b0 + b) * n_A + zc[u]];
#pragma unroll
                for (int v = 0; v < V; ++v) acc[b][v] = fmaf(zb, f[v], acc[b][v]);
              }
            }
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

// Chunks of live rows for the down-projection: about 1024 blocks of 4 waves,
// at least 16 rows per chunk, and partial sums kept under ~1/4 of the bytes
// of the rows themselves.
static int down_chunks_wanted(int n_live, int B, int d, int vec) {
  const int col_blocks = (d + 64 * vec - 1) / (64 * vec);
  int want = (1024 + col_blocks - 1) / col_blocks;
  const int by_rows = (n_live + 15) / 16;
  const int by_bytes = B > 0 ? (n_live + 8 * B - 1) / (8 * B) : want;
  if (want > by_rows) want = by_rows;
  if (want > by_bytes) want = by_bytes;
  if (want > 256) want = 256;
  if (want < 1) want = 1;
  return want;
}

static DownPlan plan_down(int n_live, int B, int d, int vec) {
  DownPlan p;
  p.col_blocks = (d + 64 * vec - 1) / (64 * vec);
  const int want = down_chunks_wanted(n_live, B, d, vec);
  p.rows_per_chunk = n_live > 0 ? (n_live + want - 1) / want : 1;
  p.n_chunks = n_live > 0 ? (n_live + p.rows_per_chunk - 1) / p.rows_per_chunk : 1;
  return p;
}

// Row chunks of the matrix-core down-projection: about `blocks` blocks over
// the 64-column slices, at least 64 and at most kDsMaxRows rows each (never
// decreasing in n, so the value at n = d_ff bounds every call).  The retained
// rows aim at POP_DOWN_BLOCKS blocks; the selected rows, whose launch waits
// for the top-k, at POP_DOWN_S_BLOCKS.
#ifndef POP_DOWN_FOLD
#define POP_DOWN_FOLD 1  // 0: the selected rows in a launch of their own
#endif
#ifndef POP_DOWN_BLOCKS
#define POP_DOWN_BLOCKS 1024
#endif
#ifndef POP_DOWN_S_BLOCKS
#define POP_DOWN_S_BLOCKS 512
#endif
static int down_mfma_chunks(int n, int d, int blocks = POP_DOWN_BLOCKS) {
  const int slices = (d + 63) / 64;
  int want = blocks / slices;  // the whole grid within the block budget
  const int by_rows = (n + kDsRows - 1) / kDsRows;
  if (want > by_rows) want = by_rows;
  const int least = (n + kDsMaxRows - 1) / kDsMaxRows;
  if (want < least) want = least;
  return want < 1 ? 1 : want;
}

// Rows per chunk and the number of (non-empty) chunks for n rows.
static void down_mfma_plan(int n, int d, int blocks, int* rows_per_chunk, int* chunks) {
  if (n <= 0) {
    *rows_per_chunk = 1;
    *chunks = 0;
    return;
  }
  const int want = down_mfma_chunks(n, d, blocks);
  *rows_per_chunk = (n + want - 1) / want;
  *chunks = (n + *rows_per_chunk - 1) / *rows_per_chunk;
}

static size_t down_ws_bytes(int32_t batch, int32_t d, int32_t n_live) {
  // The chunk count only grows with n_live; bf16 (fewer column blocks) wants at least as many as fp32.
  const int c8 = down_chunks_wanted(n_live, batch, d, 8);
  const int c4 = down_chunks_wanted(n_live, batch, d, 4);
  const int cm = down_mfma_chunks(n_live, d) + down_mfma_chunks(n_live, d, POP_DOWN_S_BLOCKS);
  int chunks = c8 > c4 ? c8 : c4;
  if (cm > chunks) chunks = cm;
  const int b = batch > 0 ? batch : 1;
  return align_up((size_t)chunks * b * d * sizeof(float), 256);
}

struct DecodeWs {
  uint32_t* ctl;  // control words of the single-launch step (zero between calls)
  float* z;
  float* score;
  int32_t* Q;    // selected positions into C
  int32_t* sel;  // selected channels
  uint64_t* hand;  // single-launch step: hand-over words (zero between calls)
  char* down;
  size_t down_bytes;
};

constexpr int kFusedRBlocks = POP_FUSED_RBLOCKS;

static size_t fused_partial_bytes(int32_t d, int32_t d_ff) {
  (void)d_ff;
  // one partial y per retained block, slice-major over whole slices
  return align_up((size_t)kFusedRBlocks * align_up((size_t)d, kFinCols) * sizeof(float), 256);
}

static_assert(kCtlBytes + kHandBytes == POP_DECODE_WS_Z_OFFSET, "z follows the control and hand-over words");

static size_t decode_ws_layout(int32_t batch, int32_t d, int32_t d_ff, char* base, DecodeWs* out) {
  const size_t tb = kCtlBytes + kHandBytes;
  const size_t zb = align_up((size_t)batch * d_ff * sizeof(float) + 16, 256);
  const size_t sb = align_up((size_t)d_ff * sizeof(float), 256);
  const size_t qb = align_up((size_t)d_ff * sizeof(int32_t), 256);
  size_t db = down_ws_bytes(batch, d, d_ff);
  if (batch == 1) {
    const size_t fb = fused_partial_bytes(d, d_ff);
    if (fb > db) db = fb;
  }
  if (out) {
    out->ctl = (uint32_t*)base;
    out->hand = (uint64_t*)(base + kCtlBytes);
    char* p = base + tb;
    out->z = (float*)p;
    out->score = (float*)(p += zb);
    out->Q = (int32_t*)(p += sb);
    out->sel = (int32_t*)(p += qb);
    out->down = p + qb;
    out->down_bytes = db;
  }
  return tb + zb + sb + 2 * qb + db;
}

// ---- stage launchers (arguments already validated)
// Batches of 2..64 rows in bf16 run on the matrix cores (16-token tiles, the
// unused token rows cost matrix-core time only, which the weight stream
// hides); fp32 and wider batches run the FMA kernels.
#ifndef POP_MFMA_MIN_BATCH
#define POP_MFMA_MIN_BATCH 2
#endif
template <typename T>
static bool use_mfma(int B) {
  return std::is_same<T, bf16s>::value && B >= POP_MFMA_MIN_BATCH && B <= 16 * kDecMaxTiles;
}

template <typename T>
static void launch_gateup(hipStream_t st, const void* x, int B, int d, const void* Wg, const void* Wu, int d_ff,
                          const int32_t* R, int n_R, const int32_t* C, int n_C, float* z, float* score) {
  const int n_A = n_R + n_C;
  if (use_mfma<T>(B)) {
    if (n_A == 0) return;
    const bool identity = R == nullptr && n_C == 0;
    const int nb = gateup_lds_blocks(n_A);
#define POP_GL(MT)                                                                                            \
  if (identity)                                                                                               \
    POP_LAUNCH((k_gateup_lds<MT, true>), dim3(nb), dim3(256), 0, st, (const bf16s*)x, B, d, (const bf16s*)Wg,  \
               (const bf16s*)Wu, d_ff, R, n_R, C, n_C, z, score, nb);                                          \
  else                                                                                                        \
    POP_LAUNCH((k_gateup_lds<MT, false>), dim3(nb), dim3(256), 0, st, (const bf16s*)x, B, d, (const bf16s*)Wg, \
               (const bf16s*)Wu, d_ff, R, n_R, C, n_C, z, score, nb)
    if (B <= 16) {
      POP_GL(1);
    } else if (B <= 32) {
      POP_GL(2);
    } else {
      POP_GL(4);
    }
#undef POP_GL
    return;
  }
  int grid = (n_A + 3) / 4;
  if (grid < 1) grid = 1;
  // R == NULL means identity rows (the dense baseline) only when there are no
  // candidate rows; with n_R == 0 R is never read.
#define POP_GATEUP(BT)                                                                                        \
  if (R == nullptr && n_C == 0)                                                                               \
    POP_LAUNCH((k_gateup<T, BT, true>), dim3(grid), dim3(256), 0, st, (const T*)x, B, d, (const T*)Wg, \
                       (const T*)Wu, d_ff, R, n_R, C, n_C, z, score);                                         \
  else                                                                                                        \
    POP_LAUNCH((k_gateup<T, BT, false>), dim3(grid), dim3(256), 0, st, (const T*)x, B, d, (const T*)Wg, \
                       (const T*)Wu, d_ff, R, n_R, C, n_C, z, score)
  if (B <= 1) {
    POP_GATEUP(1);
  } else if (B <= 2) {
    POP_GATEUP(2);
  } else {
    POP_GATEUP(4);
  }
#undef POP_GATEUP
}

static void launch_select(hipStream_t st, const float* score, int n_C, const int32_t* C, int k, int32_t* Q,
                          int32_t* selected) {
  if (n_C > 0)
    POP_LAUNCH(k_topk, dim3(1), dim3(kTopkThreads), topk_lds_bytes<kTopkThreads>(n_C), st, score, n_C, k, C, Q,
               selected);
}

// The down-projection over the live rows (R, then the selected rows).  With
// score set, the candidate top-k runs first: it writes topk_Q and topk_sel,
// which must then be the positions and channels the down stage reads (Q and
// sel).  On the matrix cores the top-k (up to 4096 candidates) shares a launch
// with the retained rows' product, and the selected rows follow.
// Blocks of `threads` threads of kernel the device holds at once (0 if the
// runtime cannot tell); cached per device and kernel.
static int resident_blocks_of(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess)
    return 0;
  return cache[key] = cus * per;
}

template <typename T>
static void launch_down(hipStream_t st, const float* z, int B, int n_A, const void* WdT, int d, int d_ff,
                        const int32_t* R, int n_R, const int32_t* sel, const int32_t* Q, int k, float* y,
                        float* partial, const float* score = nullptr, const int32_t* C = nullptr, int n_C = 0,
                        int32_t* topk_Q = nullptr, int32_t* topk_sel = nullptr, const DecodeWs* lw = nullptr) {
  const bool topk = score != nullptr && n_C > 0 && k > 0;
  if (B == 0) {
    if (topk) launch_select(st, score, n_C, C, k, topk_Q, topk_sel);
    return;
  }
  const int n_live = n_R + k;
  if (use_mfma<T>(B) && n_live > 0) {
    const bool identity = R == nullptr && k == 0;
    const bool topk_in = topk && n_C <= 4096;
    // the retained rows' launch: every block resident at once (the top-k
    // block included), so that no block starts after others have finished
    const int MTs = B <= 16 ? 1 : B <= 32 ? 2 : 4;
    const void* kr = MTs == 1 ? reinterpret_cast<const void*>(&k_down_stream<1, false, 2>)
                   : MTs == 2 ? reinterpret_cast<const void*>(&k_down_stream<2, false, 2>)
                              : reinterpret_cast<const void*>(&k_down_stream<4, false, 2>);
    int budget = resident_blocks_of(kr, 256);
    if (budget <= 0 || budget > POP_DOWN_BLOCKS) budget = POP_DOWN_BLOCKS;
    int rpcR, nRc, rpcS, nSc;
    down_mfma_plan(n_R, d, budget - (topk_in ? 1 : 0), &rpcR, &nRc);
    down_mfma_plan(k, d, POP_DOWN_S_BLOCKS, &rpcS, &nSc);
    const int ncol = (d + 63) / 64;
    if (topk && !topk_in) launch_select(st, score, n_C, C, k, topk_Q, topk_sel);
    const int nb0 = topk_in ? 1 : 0;
    // The selected rows join the retained rows' launch: each chunk adds the
    // selected candidates of its share of C.  With the top-k in the launch
    // (and the decode workspace's hand-over words at hand) the top-k block
    // hands the cut over inside it (PHASE 2); with the selection given, the
    // chunks read it from the list (PHASE 3): the same sums either way.
    const int n_Cs = n_A - n_R;
    const bool shares_fit = !identity && k > 0 && nRc > 0 && nRc <= 64 && n_Cs > 0 &&
                            (n_Cs + nRc - 1) / nRc <= kDsMaxRows;
    const bool fold = POP_DOWN_FOLD && shares_fit && topk_in && lw != nullptr;
    const bool given = POP_DOWN_FOLD && shares_fit && !topk_in;
    const CutLink link = fold ? CutLink{lw->hand + kLinkedTopkMaxN, lw->ctl + kCtlErr, kThrCopies, kThrStride,
                                        kPollLimit}
                              : CutLink{nullptr, nullptr, 0, 0, 0};
#define POP_DN_MFMA(MT, ID, PH, grid, rb, re, rpc, cb, nb)                                                        \
  POP_LAUNCH((k_down_stream<MT, ID, PH>), dim3(grid), dim3(256), 0, st, z, n_A, B, (const bf16s*)WdT, d, d_ff, R, \
             n_R, sel, Q, rb, re, rpc, cb, partial, nb, score, n_C, k, C, topk_Q, topk_sel, link)
#define POP_DN_MFMA_MT(...)      \
  if (B <= 16) {                 \
    POP_DN_MFMA(1, __VA_ARGS__); \
  } else if (B <= 32) {          \
    POP_DN_MFMA(2, __VA_ARGS__); \
  } else {                       \
    POP_DN_MFMA(4, __VA_ARGS__); \
  }
    if (identity) {
      POP_DN_MFMA_MT(true, 0, ncol * nRc, 0, n_R, rpcR, 0, 0)
    } else if (fold) {
      POP_DN_MFMA_MT(false, 2, 1 + ncol * nRc, 0, n_R, rpcR, 0, 1)
    } else if (given) {
      POP_DN_MFMA_MT(false, 3, ncol * nRc, 0, n_R, rpcR, 0, 0)
    } else {
      if (nb0 + nRc > 0) {
        POP_DN_MFMA_MT(false, 1, nb0 + ncol * nRc, 0, n_R, rpcR, 0, nb0)
      }
      if (nSc > 0) {
        POP_DN_MFMA_MT(false, 0, ncol * nSc, n_R, n_live, rpcS, nRc, 0)
      }
    }
#undef POP_DN_MFMA_MT
#undef POP_DN_MFMA
    const int64_t n_out = (int64_t)B * d;
    const int nch = fold || given ? nRc : nRc + nSc;
    const dim3 sgrid((unsigned)((n_out + 255) / 256));
    // the cut's words go back to zero once the launch that read them is done
    uint64_t* rst = fold ? link.thr : nullptr;
    const int nrst = fold ? kThrCopies : 0;
    if (nch <= 16) {
      POP_LAUNCH(k_sum_few<16>, sgrid, dim3(256), 0, st, (const float*)partial, nch, n_out, y, rst, nrst, kThrStride);
    } else if (nch <= 32) {
      POP_LAUNCH(k_sum_few<32>, sgrid, dim3(256), 0, st, (const float*)partial, nch, n_out, y, rst, nrst, kThrStride);
    } else if (nch <= 64) {
      POP_LAUNCH(k_sum_few<64>, sgrid, dim3(256), 0, st, (const float*)partial, nch, n_out, y, rst, nrst, kThrStride);
    } else {
      POP_LAUNCH(k_sum_chunks<0>, dim3((unsigned)((n_out + 31) / 32)), dim3(1024), 0, st, (const float*)partial, nch,
                 n_out, y, (unsigned int*)nullptr, 0);
    }
    return;
  }
  if (topk) launch_select(st, score, n_C, C, k, topk_Q, topk_sel);
  const DownPlan p = plan_down(n_live, B, d, Vec<T>::N);
  // Identity rows only for the dense baseline (no selected rows).
#define POP_DOWN(BT)                                                                                          \
  if (R == nullptr && k == 0)                                                                                 \
    POP_LAUNCH((k_down_partial<T, BT, true>), dim3(p.col_blocks, p.n_chunks), dim3(256), 0, st, z, n_A, \
                       B, (const T*)WdT, d, d_ff, R, n_R, sel, Q, n_R, n_live, p.rows_per_chunk, partial);  \
  else                                                                                                        \
    POP_LAUNCH((k_down_partial<T, BT, false>), dim3(p.col_blocks, p.n_chunks), dim3(256), 0, st, z,    \
                       n_A, B, (const T*)WdT, d, d_ff, R, n_R, sel, Q, n_R, n_live, p.rows_per_chunk, partial)
  if (B <= 1) {
    POP_DOWN(1);
  } else if (B <= 2) {
    POP_DOWN(2);
  } else {
    POP_DOWN(4);
  }
#undef POP_DOWN
  const int64_t n_out = (int64_t)B * d;
  POP_LAUNCH(k_sum_chunks<0>, dim3((unsigned)((n_out + 31) / 32)), dim3(1024), 0, st, (const float*)partial,
                     n_live > 0 ? p.n_chunks : 0, n_out, y, (unsigned int*)nullptr, 0);
}

// Batch-1 decode step in three launches of k_pop_step / k_pop_finish (for
// shapes the single-launch step does not take): false when d is too wide for
// the kernel's per-thread columns (the caller then runs the stage kernels).
template <typename T>
static bool launch_fused(hipStream_t st, const void* x, int d, const void* Wg, const void* Wu, const void* WdT,
                         int d_ff, const int32_t* R, int n_R, const int32_t* C, int n_C, int k, float* y,
                         const DecodeWs& w, bool accumulate = false, MemAdd ma = MemAdd{}) {
  constexpr int V = Vec<T>::N;
  const int nv = (d + kFusedThreads * V - 1) / (kFusedThreads * V);
  if (nv > 4) return false;
  const bool identity = (R == nullptr);
  int nbC = 0, rows_per_cblock = 1;
  if (n_C > 0) {
    nbC = (n_C + POP_FUSED_CROWS - 1) / POP_FUSED_CROWS;
    rows_per_cblock = (n_C + nbC - 1) / nbC;
    nbC = (n_C + rows_per_cblock - 1) / rows_per_cblock;
  }
  int nbR = 0, rows_per_rblock = 1;
  if (n_R > 0) {
    nbR = (n_R + 7) / 8;
    if (nbR > kFusedRBlocks) nbR = kFusedRBlocks;
    rows_per_rblock = (n_R + nbR - 1) / nbR;
    nbR = (n_R + rows_per_rblock - 1) / rows_per_rblock;
  }
  if (rows_per_cblock > kFusedMaxRows || rows_per_rblock > kFusedMaxRows) return false;
  const bool fuse_topk = n_C > 0 && k > 0 && n_C <= kFusedTopkMaxN;
  // retained shares of the two launches
  const int nbR2 = fuse_topk ? nbR * POP_SPLIT_B / 100 : 0;
  const int nbR1 = nbR - nbR2;
  float* partial = (float*)w.down;
  auto step = [&](int phase, hipStream_t sx, int nb0, int rb_base, int n_ret) {
    if (nb0 + n_ret <= 0) return;
    const dim3 grid(nb0 + n_ret);
#define POP_STEP(NVT, ID, PH)                                                                                   \
  POP_LAUNCH((k_pop_step<T, NVT, ID, PH>), grid, dim3(kFusedThreads), 0, sx, (const T*)x, (const T*)Wg,          \
             (const T*)Wu, (const T*)WdT, R, C, w.z, w.score, w.Q, w.sel, partial, d, d_ff, n_R, n_C, k,         \
             rows_per_cblock, rows_per_rblock, nb0, rb_base, nbR)
#define POP_STEP_PH(NVT, ID)   \
  if (nb0 == 0) {              \
    POP_STEP(NVT, ID, 0);      \
  } else if (phase == 1) {     \
    POP_STEP(NVT, ID, 1);      \
  } else {                     \
    POP_STEP(NVT, ID, 2);      \
  }
#define POP_STEP_ID(NVT)         \
  if (identity) {                \
    POP_STEP_PH(NVT, true)       \
  } else {                       \
    POP_STEP_PH(NVT, false)      \
  }
    if (nv <= 1) {
      POP_STEP_ID(1)
    } else if (nv <= 2) {
      POP_STEP_ID(2)
    } else {
      POP_STEP_ID(4)
    }
#undef POP_STEP_ID
#undef POP_STEP_PH
#undef POP_STEP
  };
  step(1, st, nbC, 0, nbR1);
  if (n_C > 0 && k > 0 && !fuse_topk) launch_select(st, w.score, n_C, C, k, w.Q, w.sel);
  step(2, st, fuse_topk ? 1 : 0, nbR1, nbR2);
  const dim3 fgrid((d + kFinCols - 1) / kFinCols);
  if (k > 0) {
    POP_LAUNCH((k_pop_finish<T, true>), fgrid, dim3(kFinThreads), 0, st, (const float*)partial, nbR,
               (const float*)w.z, n_R, n_R + n_C, (const int32_t*)w.sel, (const int32_t*)w.Q, k, (const T*)WdT, d,
               d_ff, y, (int)accumulate, (uint64_t*)nullptr, 0, MemAdd{});
  } else {
    if (ma.mem != nullptr)
      POP_LAUNCH((k_pop_finish<T, false, true>), fgrid, dim3(kFinThreads), 0, st, (const float*)partial, nbR,
                 (const float*)w.z, n_R, n_R + n_C, (const int32_t*)w.sel, (const int32_t*)w.Q, 0, (const T*)WdT, d,
                 d_ff, y, (int)accumulate, (uint64_t*)nullptr, 0, ma);
    else
      POP_LAUNCH((k_pop_finish<T, false>), fgrid, dim3(kFinThreads), 0, st, (const float*)partial, nbR,
                 (const float*)w.z, n_R, n_R + n_C, (const int32_t*)w.sel, (const int32_t*)w.Q, 0, (const T*)WdT, d,
                 d_ff, y, (int)accumulate, (uint64_t*)nullptr, 0, MemAdd{});
  }
  return true;
}

// Workgroups of `kernel` (kFusedThreads threads) the current device holds at
// once: its compute units times the occupancy per unit (cached per device and
// kernel; device attributes only, no stream work).
static int resident_blocks(const void* kernel) { return resident_blocks_of(kernel, kFusedThreads); }

// The batch-1 step as k_pop_linked + k_pop_finish.  Returns false, having
// launched nothing, when the step has no candidate top-k (no candidates, or
// k = 0) or does not fit (d wider than four 16-byte vectors per thread, more
// than kLinkedTopkMaxN candidates, too many rows per worker); the caller then
// takes launch_fused.
template <typename T>
static bool launch_linked(hipStream_t st, const void* x, int d, const void* Wg, const void* Wu, const void* WdT,
                          int d_ff, const int32_t* R, int n_R, const int32_t* C, int n_C, int k, float* y,
                          const DecodeWs& w, int32_t* sel_out, bool accumulate, float* mem = nullptr,
                          int32_t* pos_out = nullptr) {
  constexpr int V = Vec<T>::N;
  const int nv = (d + kFusedThreads * V - 1) / (kFusedThreads * V);
  // Without candidates there is no chain to overlap: the retained-only
  // k_pop_step (fewer registers) measured faster for the dense and static steps.
  if (nv > 4 || n_C <= 0 || k <= 0 || n_C > kLinkedTopkMaxN || n_R + n_C <= 0) return false;
  const bool identity = R == nullptr;
  const void* kern = nullptr;
#define POP_LINKED_PICK(NVT)                                                                   \
  kern = identity ? reinterpret_cast<const void*>(&k_pop_linked<T, NVT, true, false>)          \
                  : (mem != nullptr ? reinterpret_cast<const void*>(&k_pop_linked<T, NVT, false, true>) \
                                    : reinterpret_cast<const void*>(&k_pop_linked<T, NVT, false, false>))
  if (nv <= 1) {
    POP_LINKED_PICK(1);
  } else if (nv <= 2) {
    POP_LINKED_PICK(2);
  } else {
    POP_LINKED_PICK(4);
  }
#undef POP_LINKED_PICK
  int cap = resident_blocks(kern) - 1;  // block 0 is the top-k
  if (cap > kLinkedMaxWorkers) cap = kLinkedMaxWorkers;
  if (cap < 1) return false;
  int nW = (n_R + n_C + 7) / 8;
  if (nW > cap) nW = cap;
  if (nW < 1) nW = 1;
  if ((n_C + nW - 1) / nW + (n_R + nW - 1) / nW > kFusedMaxRows) return false;
  const dim3 grid(1 + nW);
  float* partial = (float*)w.down;
#define POP_LINKED(NVT, ID, MEM)                                                                                         \
  POP_LAUNCH((k_pop_linked<T, NVT, ID, MEM>), grid, dim3(kFusedThreads), 0, st, (const T*)x, (const T*)Wg,              \
             (const T*)Wu, (const T*)WdT, R, C, w.z, w.score, w.hand, sel_out, partial, w.ctl,                     \
             w.hand + kPairsWord, d, d_ff, n_R, n_C, k, nW, mem, pos_out)
#define POP_LINKED_ID(NVT)        \
  if (identity) {                 \
    POP_LINKED(NVT, true, false);  \
  } else if (mem != nullptr) {    \
    POP_LINKED(NVT, false, true);  \
  } else {                        \
    POP_LINKED(NVT, false, false); \
  }
  if (nv <= 1) {
    POP_LINKED_ID(1)
  } else if (nv <= 2) {
    POP_LINKED_ID(2)
  } else {
    POP_LINKED_ID(4)
  }
#undef POP_LINKED_ID
#undef POP_LINKED
  POP_LAUNCH((k_pop_finish<T, false>), dim3((d + kFinCols - 1) / kFinCols), dim3(kFinThreads), 0, st,
             (const float*)partial, nW, (const float*)w.z, n_R, n_R + n_C, (const int32_t*)w.sel,
             (const int32_t*)w.Q, 0, (const T*)WdT, d, d_ff, y, (int)accumulate, w.hand, (int)kHandWords, MemAdd{});
  return true;
}

// The fused path's launch conditions (launch_fused returns false, before any
// launch, when they fail).
template <typename T>
static bool fused_fits(int d, int n_R, int n_C) {
  constexpr int V = Vec<T>::N;
  if ((d + kFusedThreads * V - 1) / (kFusedThreads * V) > 4) return false;
  const int nbC = n_C > 0 ? (n_C + POP_FUSED_CROWS - 1) / POP_FUSED_CROWS : 0;
  if (nbC > 0 && (n_C + nbC - 1) / nbC > kFusedMaxRows) return false;
  int nbR = n_R > 0 ? (n_R + 7) / 8 : 0;
  if (nbR > kFusedRBlocks) nbR = kFusedRBlocks;
  if (nbR > 0 && (n_R + nbR - 1) / nbR > kFusedMaxRows) return false;
  return true;
}

static pop_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}

// ---- validation
static pop_status check_shape(int32_t batch, int32_t d, int32_t d_ff, pop_dtype dt) {
  pop_status s = check_dtype_width(dt, d);
  if (s != POP_OK) return s;
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (batch < 0 || batch > POP_MAX_BATCH) return fail(POP_ERR_BAD_SHAPE, "batch=%d outside [0, %d]", batch, POP_MAX_BATCH);
  return POP_OK;
}

static pop_status check_lists(int32_t d_ff, const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C,
                              bool r_may_be_identity, void* stream) {
  if (n_R < 0 || n_C < 0 || (int64_t)n_R + n_C > d_ff)
    return fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, n_C=%d inconsistent with d_ff=%d", n_R, n_C, d_ff);
  if ((n_R > 0 && R == nullptr && !r_may_be_identity) || (n_C > 0 && C == nullptr))
    return fail(POP_ERR_INVALID_ARGUMENT, "R or C is NULL with a nonzero size");
  if (R == nullptr && r_may_be_identity && n_C > 0 && n_R > 0)
    return fail(POP_ERR_INVALID_ARGUMENT, "R == NULL (identity) is only valid with n_C == 0");
  if (kDebugLists) return debug_check_device_lists(R, n_R, C, n_C, d_ff, stream);
  return POP_OK;
}

pop_status debug_check_device_lists(const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, int32_t d_ff,
                                    void* stream) {
  if (debug_nesting() > 0) return POP_OK;  // the outer entry point checked its own lists
  // the copies go on the caller's stream, behind whatever wrote the lists
  std::vector<int32_t> hr(R != nullptr && n_R > 0 ? n_R : 0), hc(C != nullptr && n_C > 0 ? n_C : 0);
  const hipStream_t h = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!hr.empty()) e = hipMemcpyAsync(hr.data(), R, hr.size() * sizeof(int32_t), hipMemcpyDeviceToHost, h);
  if (e == hipSuccess && !hc.empty()) e = hipMemcpyAsync(hc.data(), C, hc.size() * sizeof(int32_t), hipMemcpyDeviceToHost, h);
  if (e == hipSuccess) e = hipStreamSynchronize(h);
  if (e != hipSuccess) return fail(POP_ERR_HIP, "debug copy of the index lists failed: %s", hipGetErrorString(e));
  return pop_check_lists(hr.empty() ? nullptr : hr.data(), (int32_t)hr.size(), hc.empty() ? nullptr : hc.data(),
                         (int32_t)hc.size(), nullptr, 0, d_ff);
}

}  // namespace pop

using namespace pop;

#define POP_DISPATCH(dt, FN, ...) \
  ((dt) == POP_BF16 ? FN<bf16s>(__VA_ARGS__) : FN<float>(__VA_ARGS__))

namespace pop {
bool decode_ffn_accumulate_b1(const void* x, int32_t d, const void* W_gate, const void* W_up, const void* W_downT,
                              int32_t d_ff, pop_dtype dt, bool dense, const int32_t* R, int32_t n_R,
                              const int32_t* C, int32_t n_C, double r, float* y, int32_t* selected, void* ws,
                              void* stream) {
  if (dense) {
    R = nullptr;
    n_R = d_ff;
    C = nullptr;
    n_C = 0;
  }
  if (n_R + n_C <= 0) return false;
  if (!(dt == POP_BF16 ? fused_fits<bf16s>(d, n_R, n_C) : fused_fits<float>(d, n_R, n_C))) return false;
  const int32_t k = dense ? 0 : topk_count(d_ff, r, n_R, n_C);
  DecodeWs w;
  decode_ws_layout(1, d, d_ff, (char*)ws, &w);
  const int32_t* Rk = dense ? nullptr : (R != nullptr ? R : w.Q);  // NULL R: identity (every channel)
  const int32_t* Ck = C != nullptr ? C : w.Q;
  DecodeWs wf = w;
  if (selected != nullptr) wf.sel = selected;
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (POP_LINKED_ON && POP_DISPATCH(dt, launch_linked, st, x, d, W_gate, W_up, W_downT, d_ff, Rk, n_R, Ck, n_C, k, y,
                                    w, selected, true))
    return true;
  return POP_DISPATCH(dt, launch_fused, st, x, d, W_gate, W_up, W_downT, d_ff, Rk, n_R, Ck, n_C, k, y, wf, true);
}

bool decode_periodic_kept_b1(const void* x, int32_t d, const void* W_gate, const void* W_up, const void* W_downT,
                             int32_t d_ff, pop_dtype dt, const int32_t* rows, int32_t n_R, int32_t k, float* memory,
                             const int32_t* positions, int32_t n_C, float* y, void* ws, void* stream) {
  const int32_t n = n_R + k;
  if (n <= 0 || rows == nullptr || k <= 0 || memory == nullptr || positions == nullptr) return false;
  if (!(dt == POP_BF16 ? fused_fits<bf16s>(d, n, 0) : fused_fits<float>(d, n, 0))) return false;
  DecodeWs w;
  decode_ws_layout(1, d, d_ff, (char*)ws, &w);
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  const MemAdd ma{memory, positions, n_R, k, n_C};
  return POP_DISPATCH(dt, launch_fused, st, x, d, W_gate, W_up, W_downT, d_ff, rows, n, (const int32_t*)nullptr, 0, 0,
                      y, w, false, ma);
}

bool decode_periodic_refresh_b1(const void* x, int32_t d, const void* W_gate, const void* W_up, const void* W_downT,
                                int32_t d_ff, pop_dtype dt, const int32_t* R, int32_t n_R, const int32_t* C,
                                int32_t n_C, int32_t k, float* memory, int32_t* positions, int32_t* selected, float* y,
                                void* ws, void* stream) {
  if (R == nullptr || n_C <= 0 || k <= 0 || memory == nullptr || positions == nullptr || selected == nullptr)
    return false;
  if (!(dt == POP_BF16 ? fused_fits<bf16s>(d, n_R, n_C) : fused_fits<float>(d, n_R, n_C))) return false;
  DecodeWs w;
  decode_ws_layout(1, d, d_ff, (char*)ws, &w);
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  return POP_LINKED_ON && POP_DISPATCH(dt, launch_linked, st, x, d, W_gate, W_up, W_downT, d_ff, R, n_R, C, n_C, k, y,
                                       w, selected, false, memory, positions);
}

float* decode_ws_z(void* ws, int32_t batch, int32_t d, int32_t d_ff) {
  DecodeWs w;
  decode_ws_layout(batch, d, d_ff, (char*)ws, &w);
  return w.z;
}
}  // namespace pop

extern "C" size_t pop_decode_workspace_bytes(int32_t batch, int32_t d, int32_t d_ff) {
  if (batch < 0 || d <= 0 || d_ff <= 0) return 0;
  return decode_ws_layout(batch, d, d_ff, nullptr, nullptr);
}

extern "C" size_t pop_decode_down_workspace_bytes(int32_t batch, int32_t d, int32_t n_live) {
  if (batch < 0 || d <= 0 || n_live < 0) return 0;
  return down_ws_bytes(batch, d, n_live > 0 ? n_live : 1);
}

extern "C" pop_status pop_decode_gateup(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                        const void* W_up, int32_t d_ff, pop_dtype dt, const int32_t* R,
                                        int32_t n_R, const int32_t* C, int32_t n_C, float* z, float* score,
                                        void* stream) {
  clear_error();
  pop_status s = check_shape(batch, d, d_ff, dt);
  if (s != POP_OK) return s;
  if ((s = check_lists(d_ff, R, n_R, C, n_C, true, stream)) != POP_OK) return s;
  if ((batch > 0 && (x == nullptr || z == nullptr)) || W_gate == nullptr || W_up == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "x, z, W_gate and W_up must be non-NULL");
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up))
    return fail(POP_ERR_MISALIGNED, "x and the weights must be 16-byte aligned");
  trace_mark(stream);
  POP_DISPATCH(dt, launch_gateup, (hipStream_t)stream, x, batch, d, W_gate, W_up, d_ff, R, n_R, C, n_C, z, score);
  return launched();
}

extern "C" pop_status pop_decode_select(const float* score, int32_t n_C, const int32_t* C, int32_t k,
                                        int32_t* positions, int32_t* selected, void* stream) {
  clear_error();
  if (n_C < 0 || n_C > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "n_C=%d outside [0, %d]", n_C, POP_MAX_D_FF);
  if (k < 0 || k > n_C) return fail(POP_ERR_INVALID_ARGUMENT, "k=%d outside [0, n_C=%d]", k, n_C);
  if (n_C > 0 && (score == nullptr || C == nullptr || (k > 0 && (positions == nullptr || selected == nullptr))))
    return fail(POP_ERR_INVALID_ARGUMENT, "score, C, positions and selected must be non-NULL");
  trace_mark(stream);
  launch_select((hipStream_t)stream, score, n_C, C, k, positions, selected);
  return launched();
}

extern "C" pop_status pop_decode_down(const float* z, int32_t batch, int32_t n_A, const void* W_downT, int32_t d,
                                      int32_t d_ff, pop_dtype dt, const int32_t* R, int32_t n_R,
                                      const int32_t* selected, const int32_t* positions, int32_t k, float* y,
                                      void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_shape(batch, d, d_ff, dt);
  if (s != POP_OK) return s;
  if (n_R < 0 || k < 0 || n_A < n_R + k || n_A > d_ff)
    return fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, k=%d, n_A=%d inconsistent (d_ff=%d)", n_R, k, n_A, d_ff);
  if ((n_R > 0 && R == nullptr && k > 0) || (k > 0 && (selected == nullptr || positions == nullptr)))
    return fail(POP_ERR_INVALID_ARGUMENT, "R, selected or positions is NULL with a nonzero size");
  if ((batch > 0 && (z == nullptr || y == nullptr)) || W_downT == nullptr || ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "z, y, W_downT and ws must be non-NULL");
  if (!aligned16(W_downT) || !aligned16(y) || !aligned16(ws))
    return fail(POP_ERR_MISALIGNED, "W_downT, y and ws must be 16-byte aligned");
  const size_t need = pop_decode_down_workspace_bytes(batch, d, n_R + k);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  trace_mark(stream);
  POP_DISPATCH(dt, launch_down, (hipStream_t)stream, z, batch, n_A, W_downT, d, d_ff, R, n_R, selected, positions, k,
               y, (float*)ws);
  return launched();
}

extern "C" pop_status pop_decode_ffn(const void* x, int32_t batch, int32_t d, const void* W_gate, const void* W_up,
                                     const void* W_downT, int32_t d_ff, pop_dtype dt, const int32_t* R, int32_t n_R,
                                     const int32_t* C, int32_t n_C, double r, float* y, int32_t* selected, void* ws,
                                     size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_shape(batch, d, d_ff, dt);
  if (s != POP_OK) return s;
  if (!(r >= 0.0 && r < 1.0)) return fail(POP_ERR_INVALID_ARGUMENT, "r=%g outside [0, 1)", r);
  if ((s = check_lists(d_ff, R, n_R, C, n_C, false, stream)) != POP_OK) return s;
  if ((batch > 0 && (x == nullptr || y == nullptr)) || W_gate == nullptr || W_up == nullptr || W_downT == nullptr ||
      ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_downT) || !aligned16(y) ||
      !aligned16(ws))
    return fail(POP_ERR_MISALIGNED, "x, weights, y and ws must be 16-byte aligned");
  const size_t need = pop_decode_workspace_bytes(batch, d, d_ff);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  const int32_t k = topk_count(d_ff, r, n_R, n_C);
  DecodeWs w;
  decode_ws_layout(batch, d, d_ff, (char*)ws, &w);
  // An empty R is passed to the kernels as a non-NULL list (NULL means identity there).
  const int32_t* Rk = R != nullptr ? R : w.Q;
  const int32_t* Ck = C != nullptr ? C : w.Q;
  hipStream_t st = (hipStream_t)stream;
  DecodeWs wf = w;
  if (selected != nullptr) wf.sel = selected;  // the top-k writes the caller's list directly
  trace_mark(st);
  if (batch == 1 && n_R + n_C > 0 &&
      ((POP_LINKED_ON && POP_DISPATCH(dt, launch_linked, st, x, d, W_gate, W_up, W_downT, d_ff, Rk, n_R, Ck, n_C, k,
                                      y, w, selected, false)) ||
       POP_DISPATCH(dt, launch_fused, st, x, d, W_gate, W_up, W_downT, d_ff, Rk, n_R, Ck, n_C, k, y, wf)))
    return launched();
  POP_DISPATCH(dt, launch_gateup, st, x, batch, d, W_gate, W_up, d_ff, Rk, n_R, Ck, n_C, w.z, w.score);
  int32_t* sel = selected != nullptr ? selected : w.sel;  // the down stage reads the selected channels here
  POP_DISPATCH(dt, launch_down, st, w.z, batch, n_R + n_C, W_downT, d, d_ff, Rk, n_R, sel, w.Q, k, y,
               (float*)w.down, w.score, Ck, n_C, w.Q, sel, &w);
  return launched();
}

extern "C" pop_status pop_dense_ffn_decode(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                           const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                           float* y, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_shape(batch, d, d_ff, dt);
  if (s != POP_OK) return s;
  if ((batch > 0 && (x == nullptr || y == nullptr)) || W_gate == nullptr || W_up == nullptr || W_downT == nullptr ||
      ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_downT) || !aligned16(y) ||
      !aligned16(ws))
    return fail(POP_ERR_MISALIGNED, "x, weights, y and ws must be 16-byte aligned");
  const size_t need = pop_decode_workspace_bytes(batch, d, d_ff);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  DecodeWs w;
  decode_ws_layout(batch, d, d_ff, (char*)ws, &w);
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (batch == 1 &&
      ((POP_LINKED_ON && POP_DISPATCH(dt, launch_linked, st, x, d, W_gate, W_up, W_downT, d_ff, nullptr, d_ff,
                                      nullptr, 0, 0, y, w, nullptr, false)) ||
       POP_DISPATCH(dt, launch_fused, st, x, d, W_gate, W_up, W_downT, d_ff, nullptr, d_ff, nullptr, 0, 0, y, w)))
    return launched();
  POP_DISPATCH(dt, launch_gateup, st, x, batch, d, W_gate, W_up, d_ff, nullptr, d_ff, nullptr, 0, w.z, nullptr);
  POP_DISPATCH(dt, launch_down, st, w.z, batch, d_ff, W_downT, d, d_ff, nullptr, d_ff, nullptr, nullptr, 0, y,
               (float*)w.down);
  return launched();
}

// ---------------------------------------------------------------- allocation-free decode step
// pop_decode_ffn with its workspace in a file-scope device array instead of a
// caller buffer, for callers that cannot allocate (graph capture, tight
// serving loops).  Every call on one GPU shares that GPU's array.
namespace pop {
constexpr size_t kScratchBytes = (size_t)POP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

// Clears n 64-bit words (the control and hand-over words must start at 0).
__global__ __launch_bounds__(256) void k_zero_u64(uint64_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // the array's device address, per device

// The current device's address of `scratch`, looked up (and its control
// words cleared, on `st`) on the first call on that device.  Host code uses
// this address, never the array's name.
pop_status device_scratch(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(POP_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(POP_ERR_HIP, "device %d beyond the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(POP_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    const int words = (int)((kCtlBytes + kHandBytes) / sizeof(uint64_t));
    hipLaunchKernelGGL(k_zero_u64, dim3((words + 255) / 256), dim3(256), 0, st, (uint64_t*)p, words);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(POP_ERR_HIP, "clearing the scratch failed: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return POP_OK;
}
}  // namespace
}  // namespace pop

extern "C" pop_status pop_decode_ffn_noalloc(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                             const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                             const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, double r,
                                             float* y, int32_t* selected, void* stream) {
  clear_error();
  pop_status s = check_shape(batch, d, d_ff, dt);
  if (s != POP_OK) return s;
  const size_t need = pop_decode_workspace_bytes(batch, d, d_ff);
  if (need > kScratchBytes)
    return fail(POP_ERR_WORKSPACE_TOO_SMALL,
                "batch=%d, d=%d, d_ff=%d needs %zu workspace bytes, beyond the %zu-byte scratch of "
                "pop_decode_ffn_noalloc; use pop_decode_ffn with a caller workspace",
                batch, d, d_ff, need, kScratchBytes);
  void* ws = nullptr;
  if ((s = device_scratch((hipStream_t)stream, &ws)) != POP_OK) return s;
  return pop_decode_ffn(x, batch, d, W_gate, W_up, W_downT, d_ff, dt, R, n_R, C, n_C, r, y, selected, ws,
                        kScratchBytes, stream);
}
