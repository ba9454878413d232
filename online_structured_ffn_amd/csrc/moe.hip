// Mixture-of-experts form of the pruned decode step.  The POP notes evaluate
// MoE models (Qwen2-57B-A14B among them) with the method applied per expert
// FFN; reading taken: each expert keeps its own R/C/P partition built from the
// prompt tokens routed to it, and in each decode step it runs the POP step
// (gate/up over its R u C, candidate score = max over the tokens routed to it,
// top-k, down over R u S) on its routed tokens; a token's output is the
// routing-weighted sum of its two experts' outputs, added in expert order.
//
// Kernels of one step (all experts in each launch, no host synchronisation):
//   k_moe_top2, k_moe_bucket   routing (moe_route.h)
//   bf16 steps of up to 64 tokens: the batched decode's matrix-core kernels in
//   their expert form (grid row = expert, its routed pairs as the tokens):
//     k_gateup_lds             z and candidate scores
//     k_down_stream            the retained rows, with each expert's top-k as
//                              one block of the launch; then the selected rows
//   otherwise:
//     k_moe_gateup             z and candidate scores, one wave per (expert, row)
//     k_moe_topk               one workgroup per expert
//     k_moe_down               (column slice, live-row chunk, expert) blocks
//   both write partial y per (chunk, routed pair), then
//   k_moe_combine              fixed-order sum over chunks, then over the two
//                              experts with their weights
// An expert that no token of the step reaches does nothing: its blocks exit at
// once and its selected list is left as it was.
#include <hip/hip_runtime.h>

#include "decode_mfma.h"
#include "moe_route.h"
#include "pop_device.h"
#include "pop_internal.h"

namespace pop {

constexpr int kMoeBT = 8;  // routed tokens per pass over a weight row

__device__ __forceinline__ int moe_channel(int ch, int d_ff) { return min(max(ch, 0), d_ff - 1); }

// ---------------------------------------------------------------- gate / up
// Block (b, e): rows 4b + wave, stepping by 4 * gridDim.x, of expert e's
// R u C.  z row of routed pair p = offsets[e] + i is z[p * n_A + row].
template <typename T>
__global__ __launch_bounds__(256) void k_moe_gateup(const T* __restrict__ x, int d, const T* __restrict__ Wg,
                                                    const T* __restrict__ Wu, int d_ff, const int32_t* __restrict__ R,
                                                    int n_R, const int32_t* __restrict__ C, int n_C,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ tokens, float* __restrict__ z,
                                                    float* __restrict__ score) {
  constexpr int V = Vec<T>::N;
  constexpr int STEP = 64 * V;
  const int e = blockIdx.y;
  const int o0 = offsets[e];
  const int cnt = offsets[e + 1] - o0;
  if (cnt <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_A = n_R + n_C;
  const int64_t wstride = (int64_t)d_ff * d;
  const int32_t* Re = R + (int64_t)e * n_R;
  const int32_t* Ce = C + (int64_t)e * n_C;
  for (int p = blockIdx.x * 4 + wave; p < n_A; p += gridDim.x * 4) {
    const int ch = moe_channel(p < n_R ? Re[p] : Ce[p - n_R], d_ff);
    const T* wg = Wg + e * wstride + (int64_t)ch * d;
    const T* wu = Wu + e * wstride + (int64_t)ch * d;
    float smax = 0.f;
    for (int b0 = 0; b0 < cnt; b0 += kMoeBT) {
      const int nb = min(kMoeBT, cnt - b0);
      const T* xr[kMoeBT];
#pragma unroll
      for (int b = 0; b < kMoeBT; ++b) xr[b] = x + (int64_t)tokens[o0 + b0 + min(b, nb - 1)] * d;
      float ag[kMoeBT], au[kMoeBT];
#pragma unroll
      for (int b = 0; b < kMoeBT; ++b) ag[b] = au[b] = 0.f;
      for (int k0 = 0; k0 < d; k0 += 2 * STEP) {
        u32x4 qg[2], qu[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int k = k0 + j * STEP + lane * V;
          if (k < d) {
            qg[j] = ld16_stream(wg + k);
            qu[j] = ld16_stream(wu + k);
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int k = k0 + j * STEP + lane * V;
          if (k < d) {
            float g[V], u[V];
            unpack(qg[j], g, T{});
            unpack(qu[j], u, T{});
#pragma unroll
            for (int b = 0; b < kMoeBT; ++b) {
              if (b < nb) {
                float xv[V];
                unpack(ld16(xr[b] + k), xv, T{});
#pragma unroll
                for (int v = 0; v < V; ++v) {
                  ag[b] = fmaf(g[v], xv[v], ag[b]);
                  au[b] = fmaf(u[v], xv[v], au[b]);
                }
              }
            }
          }
        }
      }
#pragma unroll
      for (int b = 0; b < kMoeBT; ++b) {
        if (b < nb) {
          const float gs = wave_sum_last(ag[b]);
          const float us = wave_sum_last(au[b]);
          const float zz = silu(gs) * us;  // exact in lane 63
          if (lane == 63) z[(int64_t)(o0 + b0 + b) * n_A + p] = zz;
          smax = fmaxf(smax, fabsf(zz));
        }
      }
    }
    if (lane == 63 && p >= n_R) score[(int64_t)e * n_C + p - n_R] = smax;
  }
}

// ---------------------------------------------------------------- top-k
template <int MAXN, int NTH>
__global__ __launch_bounds__(NTH) void k_moe_topk(const float* __restrict__ score, int n_C, int k,
                                                  const int32_t* __restrict__ C, const int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ Q, int32_t* __restrict__ S) {
  extern __shared__ __align__(16) unsigned char topk_smem[];  // topk_lds_bytes<NTH>(n_C)
  const int e = blockIdx.x;
  if (offsets[e + 1] == offsets[e]) return;
  topk_select<NTH>(score + (int64_t)e * n_C, n_C, k, C + (int64_t)e * n_C, Q + (int64_t)e * k, S + (int64_t)e * k,
                   topk_smem);
}

// ---------------------------------------------------------------- down
// Block (cs, c, e): columns cs * 64 * V + [0, 64 * V) of the live rows
// [c * rows_per_chunk, ...) of expert e (R first, then S).  Wave w takes rows
// q0 + w, q0 + w + 4, ...; the four wave sums are added in wave order and
// written to partial[c][p][:] for each routed pair p of the expert.
template <typename T>
__global__ __launch_bounds__(256) void k_moe_down(const float* __restrict__ z, int n_A, const T* __restrict__ WdT,
                                                  int d, int d_ff, const int32_t* __restrict__ R, int n_R,
                                                  const int32_t* __restrict__ S, const int32_t* __restrict__ Q, int k,
                                                  const int32_t* __restrict__ offsets, int rows_per_chunk, int n_pairs,
                                                  float* __restrict__ partial) {
  constexpr int V = Vec<T>::N;
  constexpr int U = 4;
  __shared__ float red[3][kMoeBT * V][64];
  const int e = blockIdx.z;
  const int o0 = offsets[e];
  const int cnt = offsets[e + 1] - o0;
  if (cnt <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (blockIdx.x * 64 + lane) * V;
  const bool on = col < d;
  const int n_live = n_R + k;
  const int q0 = blockIdx.y * rows_per_chunk;
  const int q1 = min(n_live, q0 + rows_per_chunk);
  const T* W = WdT + (int64_t)e * d_ff * d;
  const int32_t* Re = R + (int64_t)e * n_R;
  const int32_t* Se = S + (int64_t)e * k;
  const int32_t* Qe = Q + (int64_t)e * k;
  for (int b0 = 0; b0 < cnt; b0 += kMoeBT) {
    const int nb = min(kMoeBT, cnt - b0);
    float acc[kMoeBT][V];
#pragma unroll
    for (int b = 0; b < kMoeBT; ++b)
#pragma unroll
      for (int v = 0; v < V; ++v) acc[b][v] = 0.f;
    for (int q = q0 + wave; q < q1; q += 4 * U) {
      u32x4 w[U];
      int zc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int qq = q + 4 * u;
        zc[u] = -1;
        if (qq < q1) {
          int ch;
          if (qq < n_R) {
            ch = Re[qq];
            zc[u] = qq;
          } else {
            ch = Se[qq - n_R];
            zc[u] = min(n_R + max(Qe[qq - n_R], 0), n_A - 1);
          }
          if (on) w[u] = ld16_stream(W + (int64_t)moe_channel(ch, d_ff) * d + col);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (zc[u] >= 0 && on) {
          float f[V];
          unpack(w[u], f, T{});
#pragma unroll
          for (int b = 0; b < kMoeBT; ++b) {
            if (b < nb) {
              const float zb = z[(int64_t)(o0 + b0 + b) * n_A + zc[u]];
#pragma unroll
              for (int v = 0; v < V; ++v) acc[b][v] = fmaf(zb, f[v], acc[b][v]);
            }
          }
        }
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int b = 0; b < kMoeBT; ++b)
#pragma unroll
        for (int v = 0; v < V; ++v) red[wave - 1][b * V + v][lane] = acc[b][v];
    }
    __syncthreads();
    if (wave == 0 && on) {
#pragma unroll
      for (int b = 0; b < kMoeBT; ++b) {
        if (b < nb) {
          float* out = partial + ((int64_t)blockIdx.y * n_pairs + o0 + b0 + b) * d + col;
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

// ---------------------------------------------------------------- combine
// y[t, col] = sum over t's two experts, lower expert id first, of
// weight * (sum over chunks, in chunk order, of partial[c][slot][col]).
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ partial, int n_chunks, int n_pairs,
                                                     int d, const int32_t* __restrict__ ex,
                                                     const float* __restrict__ wt, const int32_t* __restrict__ slot,
                                                     float* __restrict__ y) {
  const int t = blockIdx.y;
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= d) return;
  const int first = ex[2 * t] < ex[2 * t + 1] ? 0 : 1;
  float acc = 0.f;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int j = jj == 0 ? first : 1 - first;
    const int p = slot[2 * t + j];
    float s = 0.f;
    for (int c = 0; c < n_chunks; ++c) s += partial[((int64_t)c * n_pairs + p) * d + col];
    acc += wt[2 * t + j] * s;
  }
  y[(int64_t)t * d + col] = acc;
}

// ---------------------------------------------------------------- host
struct MoeDownPlan {
  int col_blocks;
  int n_chunks;
  int rows_per_chunk;
};

// About 1024 blocks over all experts, at least 16 live rows per chunk.
static MoeDownPlan plan_moe_down(int n_live, int d, int E, int vec) {
  MoeDownPlan p;
  p.col_blocks = (d + 64 * vec - 1) / (64 * vec);
  int want = (1024 + E * p.col_blocks - 1) / (E * p.col_blocks);
  const int by_rows = (n_live + 15) / 16;
  if (want > by_rows) want = by_rows;
  if (want < 1) want = 1;
  p.rows_per_chunk = n_live > 0 ? (n_live + want - 1) / want : 1;
  p.n_chunks = n_live > 0 ? (n_live + p.rows_per_chunk - 1) / p.rows_per_chunk : 1;
  return p;
}

struct MoeDecodeWs {
  int32_t* ex;
  float* wt;
  int32_t* offsets;
  int32_t* tokens;
  int32_t* slot;
  float* z;
  float* score;
  int32_t* Q;
  int32_t* S;
  float* partial;
  size_t bytes;
};

// Row chunks of the matrix-core down-projection for one expert: about 1024
// blocks over all experts and 64-column slices, 64 to kDsMaxRows rows each
// (never decreasing in n, so the value at n = d_ff bounds every call).
static int moe_mfma_chunks(int n, int d, int E) {
  const int slices = (d + 63) / 64;
  int want = (1024 + E * slices - 1) / (E * slices);
  const int by_rows = (n + kDsRows - 1) / kDsRows;
  if (want > by_rows) want = by_rows;
  const int least = (n + kDsMaxRows - 1) / kDsMaxRows;
  if (want < least) want = least;
  return want < 1 ? 1 : want;
}

// Layout for n_tokens routed tokens; sized for the widest plan (bf16 vectors,
// every channel live) so that one size serves every dtype and rate.
static MoeDecodeWs moe_decode_ws(int32_t n_tokens, int32_t d, int32_t d_ff, int32_t E, char* base) {
  const int64_t pairs = 2 * (int64_t)(n_tokens > 0 ? n_tokens : 1);
  // Every plan has n_chunks <= its wanted count, which is largest for bf16
  // (fewer column blocks) before the per-row cap: a bound for every n_live.
  const int cb8 = (d + 64 * 8 - 1) / (64 * 8);
  int chunks = (1024 + E * cb8 - 1) / (E * cb8);
  // the matrix-core plan: retained and selected rows chunked apart
  const int mc = 2 * moe_mfma_chunks(d_ff, d, E);
  if (mc > chunks) chunks = mc;
  MoeDecodeWs w;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* ptr = base ? base + o : nullptr;
    o += align_up(bytes, 256);
    return ptr;
  };
  w.ex = (int32_t*)take(pairs * 4);
  w.wt = (float*)take(pairs * 4);
  w.offsets = (int32_t*)take((size_t)(E + 1) * 4);
  w.tokens = (int32_t*)take(pairs * 4);
  w.slot = (int32_t*)take(pairs * 4);
  w.z = (float*)take((size_t)pairs * d_ff * 4);
  w.score = (float*)take((size_t)E * d_ff * 4);
  w.Q = (int32_t*)take((size_t)E * d_ff * 4);
  w.S = (int32_t*)take((size_t)E * d_ff * 4);
  w.partial = (float*)take((size_t)chunks * pairs * d * 4);
  w.bytes = o;
  return w;
}

static pop_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}

static void launch_route(hipStream_t st, const float* logits, int T, int E, int32_t* ex, float* wt,
                         int32_t* offsets, int32_t* tokens, int32_t* slot) {
  POP_LAUNCH(k_moe_top2<0>, dim3((T + 255) / 256), dim3(256), 0, st, logits, T, E, ex, wt);
  POP_LAUNCH(k_moe_bucket<0>, dim3(1), dim3(kBucketThreads), 0, st, (const int32_t*)ex, T, E, offsets, tokens,
             slot);
}

// bf16 steps of up to 64 tokens on the matrix cores (see the top of the file).
template <int MT>
static void launch_moe_decode_mfma(hipStream_t st, const void* x, int Tn, int d, int E, const void* Wg,
                                   const void* Wu, const void* WdT, int d_ff, const int32_t* R, int n_R,
                                   const int32_t* C, int n_C, int k, int32_t* S, const MoeDecodeWs& w) {
  const int n_A = n_R + n_C, n_pairs = 2 * Tn, n_live = n_R + k;
  const MoeRows mr{w.offsets, w.tokens, (int64_t)d_ff * d};
  if (n_A > 0) {
    const int nb = (n_A + kGlRows - 1) / kGlRows;
    POP_LAUNCH((k_gateup_lds<MT, false, true>), dim3(nb, E), dim3(256), 0, st, (const bf16s*)x, Tn, d,
               (const bf16s*)Wg, (const bf16s*)Wu, d_ff, R, n_R, C, n_C, w.z, w.score, nb, mr);
  }
  const int ncol = (d + 63) / 64;
  const int nRc = n_R > 0 ? moe_mfma_chunks(n_R, d, E) : 0, nSc = k > 0 ? moe_mfma_chunks(k, d, E) : 0;
  const int rpcR = nRc > 0 ? (n_R + nRc - 1) / nRc : 1, rpcS = nSc > 0 ? (k + nSc - 1) / nSc : 1;
  const int usedR = nRc > 0 ? (n_R + rpcR - 1) / rpcR : 0, usedS = nSc > 0 ? (k + rpcS - 1) / rpcS : 0;
  const bool topk = n_C > 0 && k > 0, topk_in = topk && n_C <= 4096;
  if (topk && !topk_in)
    POP_LAUNCH((k_moe_topk<kSelMaxN, 1024>), dim3(E), dim3(1024), topk_lds_bytes<1024>(n_C), st,
               (const float*)w.score, n_C, k, C, (const int32_t*)w.offsets, w.Q, S);
  const int nb0 = topk_in ? 1 : 0;
  if (nb0 + usedR > 0)
    POP_LAUNCH((k_down_stream<MT, false, 1, true>), dim3(nb0 + ncol * usedR, E), dim3(256), 0, st,
               (const float*)w.z, n_A, n_pairs, (const bf16s*)WdT, d, d_ff, R, n_R, (const int32_t*)S,
               (const int32_t*)w.Q, 0, n_R, rpcR, 0, w.partial, nb0, (const float*)w.score, n_C, k, C, w.Q, S,
               CutLink{nullptr, nullptr, 0, 0, 0}, mr);
  if (usedS > 0)
    POP_LAUNCH((k_down_stream<MT, false, 0, true>), dim3(ncol * usedS, E), dim3(256), 0, st, (const float*)w.z,
               n_A, n_pairs, (const bf16s*)WdT, d, d_ff, R, n_R, (const int32_t*)S, (const int32_t*)w.Q, n_R, n_live,
               rpcS, usedR, w.partial, 0, (const float*)nullptr, n_C, k, C, w.Q, S, CutLink{nullptr, nullptr, 0, 0, 0},
               mr);
  (void)n_live;
}

template <typename T>
static void launch_moe_decode(hipStream_t st, const void* x, int Tn, int d, const float* logits, int E,
                              const void* Wg, const void* Wu, const void* WdT, int d_ff, const int32_t* R, int n_R,
                              const int32_t* C, int n_C, int k, float* y, int32_t* S, const MoeDecodeWs& w) {
  const int n_A = n_R + n_C;
  const int n_pairs = 2 * Tn;
  launch_route(st, logits, Tn, E, w.ex, w.wt, w.offsets, w.tokens, w.slot);
  if (std::is_same<T, bf16s>::value && Tn <= 16 * kDecMaxTiles) {
    if (Tn <= 16)
      launch_moe_decode_mfma<1>(st, x, Tn, d, E, Wg, Wu, WdT, d_ff, R, n_R, C, n_C, k, S, w);
    else if (Tn <= 32)
      launch_moe_decode_mfma<2>(st, x, Tn, d, E, Wg, Wu, WdT, d_ff, R, n_R, C, n_C, k, S, w);
    else
      launch_moe_decode_mfma<4>(st, x, Tn, d, E, Wg, Wu, WdT, d_ff, R, n_R, C, n_C, k, S, w);
    const int nRc = n_R > 0 ? moe_mfma_chunks(n_R, d, E) : 0, nSc = k > 0 ? moe_mfma_chunks(k, d, E) : 0;
    const int rpcR = nRc > 0 ? (n_R + nRc - 1) / nRc : 1, rpcS = nSc > 0 ? (k + nSc - 1) / nSc : 1;
    const int used = (nRc > 0 ? (n_R + rpcR - 1) / rpcR : 0) + (nSc > 0 ? (k + rpcS - 1) / rpcS : 0);
    POP_LAUNCH(k_moe_combine, dim3((d + 255) / 256, Tn), dim3(256), 0, st, (const float*)w.partial, used, n_pairs,
               d, (const int32_t*)w.ex, (const float*)w.wt, (const int32_t*)w.slot, y);
    return;
  }
  if (n_A > 0)
    POP_LAUNCH(k_moe_gateup<T>, dim3((n_A + 3) / 4, E), dim3(256), 0, st, (const T*)x, d, (const T*)Wg,
               (const T*)Wu, d_ff, R, n_R, C, n_C, (const int32_t*)w.offsets, (const int32_t*)w.tokens, w.z, w.score);
  if (n_C > 0 && k > 0) {
    if (n_C <= 4096)
      POP_LAUNCH((k_moe_topk<4096, 256>), dim3(E), dim3(256), topk_lds_bytes<256>(n_C), st, (const float*)w.score,
                 n_C, k, C, (const int32_t*)w.offsets, w.Q, S);
    else
      POP_LAUNCH((k_moe_topk<kSelMaxN, 1024>), dim3(E), dim3(1024), topk_lds_bytes<1024>(n_C), st,
                 (const float*)w.score, n_C, k, C, (const int32_t*)w.offsets, w.Q, S);
  }
  const int n_live = n_R + k;
  const MoeDownPlan p = plan_moe_down(n_live, d, E, Vec<T>::N);
  if (n_live > 0)
    POP_LAUNCH(k_moe_down<T>, dim3(p.col_blocks, p.n_chunks, E), dim3(256), 0, st, (const float*)w.z, n_A,
               (const T*)WdT, d, d_ff, R, n_R, (const int32_t*)S, (const int32_t*)w.Q, k, (const int32_t*)w.offsets,
               p.rows_per_chunk, n_pairs, w.partial);
  POP_LAUNCH(k_moe_combine, dim3((d + 255) / 256, Tn), dim3(256), 0, st, (const float*)w.partial,
             n_live > 0 ? p.n_chunks : 0, n_pairs, d, (const int32_t*)w.ex, (const float*)w.wt,
             (const int32_t*)w.slot, y);
}

static pop_status check_experts(int32_t E) {
  if (E < 2 || E > kMoeMaxExperts) return fail(POP_ERR_BAD_SHAPE, "n_experts=%d outside [2, %d]", E, kMoeMaxExperts);
  return POP_OK;
}

}  // namespace pop

using namespace pop;

extern "C" pop_status pop_moe_route_top2(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t* experts,
                                         float* weights, int32_t* offsets, int32_t* tokens, int32_t* slots,
                                         void* stream) {
  clear_error();
  pop_status s = check_experts(n_experts);
  if (s != POP_OK) return s;
  if (n_tokens < 0 || n_tokens > POP_MAX_MOE_TOKENS)
    return fail(POP_ERR_BAD_SHAPE, "n_tokens=%d outside [0, %d]", n_tokens, POP_MAX_MOE_TOKENS);
  if (offsets == nullptr || (n_tokens > 0 && (logits == nullptr || experts == nullptr || weights == nullptr ||
                                              tokens == nullptr || slots == nullptr)))
    return fail(POP_ERR_INVALID_ARGUMENT, "an input or output pointer is NULL");
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (n_tokens > 0)
    POP_LAUNCH(k_moe_top2<0>, dim3((n_tokens + 255) / 256), dim3(256), 0, st, logits, (int)n_tokens, (int)n_experts,
               experts, weights);
  POP_LAUNCH(k_moe_bucket<0>, dim3(1), dim3(kBucketThreads), 0, st, (const int32_t*)experts, (int)n_tokens,
             (int)n_experts, offsets, tokens, slots);
  return launched();
}

extern "C" size_t pop_moe_decode_workspace_bytes(int32_t n_tokens, int32_t d, int32_t d_ff, int32_t n_experts) {
  if (n_tokens < 0 || d <= 0 || d_ff <= 0 || n_experts < 2 || n_experts > kMoeMaxExperts) return 0;
  return moe_decode_ws(n_tokens, d, d_ff, n_experts, nullptr).bytes;
}

extern "C" pop_status pop_moe_decode_ffn(const void* x, int32_t n_tokens, int32_t d, const float* logits,
                                         int32_t n_experts, const void* W_gate, const void* W_up, const void* W_downT,
                                         int32_t d_ff, pop_dtype dt, const int32_t* R, int32_t n_R, const int32_t* C,
                                         int32_t n_C, double r, float* y, int32_t* selected, void* ws,
                                         size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_dtype_width(dt, d);
  if (s != POP_OK) return s;
  if ((s = check_experts(n_experts)) != POP_OK) return s;
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (n_tokens < 0 || n_tokens > POP_MAX_BATCH)
    return fail(POP_ERR_BAD_SHAPE, "n_tokens=%d outside [0, %d]", n_tokens, POP_MAX_BATCH);
  if (!(r >= 0.0 && r < 1.0)) return fail(POP_ERR_INVALID_ARGUMENT, "r=%g outside [0, 1)", r);
  if (n_R < 0 || n_C < 0 || (int64_t)n_R + n_C > d_ff)
    return fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, n_C=%d inconsistent with d_ff=%d", n_R, n_C, d_ff);
  if ((n_R > 0 && R == nullptr) || (n_C > 0 && C == nullptr) || W_gate == nullptr || W_up == nullptr ||
      W_downT == nullptr || ws == nullptr || (n_tokens > 0 && (x == nullptr || y == nullptr || logits == nullptr)))
    return fail(POP_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_downT) || !aligned16(y) ||
      !aligned16(ws) || !aligned16(logits))
    return fail(POP_ERR_MISALIGNED, "x, logits, weights, y and ws must be 16-byte aligned");
  const MoeDecodeWs w0 = moe_decode_ws(n_tokens, d, d_ff, n_experts, nullptr);
  if (ws_bytes < w0.bytes) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, w0.bytes);
  if (n_tokens == 0) return POP_OK;
  const MoeDecodeWs w = moe_decode_ws(n_tokens, d, d_ff, n_experts, (char*)ws);
  const int32_t k = topk_count(d_ff, r, n_R, n_C);
  int32_t* S = selected != nullptr ? selected : w.S;
  // Empty lists are passed as non-NULL pointers (never read).
  const int32_t* Rk = R != nullptr ? R : w.Q;
  const int32_t* Ck = C != nullptr ? C : w.Q;
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (dt == POP_BF16)
    launch_moe_decode<bf16s>(st, x, n_tokens, d, logits, n_experts, W_gate, W_up, W_downT, d_ff, Rk, n_R, Ck, n_C, k,
                             y, S, w);
  else
    launch_moe_decode<float>(st, x, n_tokens, d, logits, n_experts, W_gate, W_up, W_downT, d_ff, Rk, n_R, Ck, n_C, k,
                             y, S, w);
  return launched();
}
