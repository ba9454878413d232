// A whole decoder layer around the pruned FFN: the attention half runs dense,
// the FFN is POP's ("POP: Online Structural Pruning ..." paper notes, "Key
// design 3" and "Limitations": attention keeps all of its parameters, only the
// FFN is pruned).  The layer is the pre-norm LLaMA layer:
//
//   h   = x + Attn(RMSNorm(x; attn_norm)) Wo_T
//   out = h + FFN(RMSNorm(h; ffn_norm))
//
// with RMSNorm (Zhang & Sennrich 2019, eq. 4), rotary embedding of q and k
// (RoFormer, Su et al. 2021, eqs. 14-15: pair (2i, 2i+1) of a head turned by
// pos * theta^(-2i/hd)), causal scaled dot-product attention (Vaswani et al.
// 2017, sec. 3.2.1) with grouped key/value heads.
//
// Kernels (all deterministic: every sum runs in a fixed order):
//   k_rmsnorm       one block per row; the output rounded to the weight dtype.
//   k_gemv_kmajor   decode projections y = x W (W K-major [K, N]): one wave per
//                   (512 or 256 columns, chunk of rows, group of tokens), fp32
//                   partial sums per row chunk.  HBM-bound: every weight byte
//                   is read once.  Its input is x itself, the RMSNorm of the
//                   residual stream computed in the wave (the q|k|v
//                   projection at batch <= 2), or the merge of the attention
//                   slices (the output projection).
//   k_gemm_decode   the same projections for 12 or more bf16 tokens on the
//                   matrix cores (256-column tiles, slices of the reduction).
//   k_qkv_rope      sums the row chunks of q|k|v, turns q and k, writes the
//                   key/value cache entries (dtype) and q (fp32).
//   k_attn_decode   one query per (sequence, head): the keys are split into
//                   64-key slices, one block each, online softmax inside the
//                   slice; (max, sum, unnormalised output) per slice.
//   k_attn_prefill  the prompt: a block per (16 queries, head, sequence) runs
//                   over 32-key tiles of the causal window in LDS.
//   k_sum_residual, k_add   the residual updates of the stream x (fp32); at
//                   batch 1 the FFN's last kernel adds its output into x instead
//                   of k_add.
// The prompt's projections use the prompt FFN's matrix-core GEMM
// (launch_gemm_kmajor).  The FFN is pop_decode_ffn / pop_dense_ffn_decode /
// pop_prefill_ffn_partition.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "pop_device.h"
#include "pop_internal.h"
#include "prompt_gemm.h"

namespace pop {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kAttnKeys = 64;       // keys per decode slice
constexpr int kPfQ = 16;            // queries per prompt-attention block
constexpr int kPfK = 32;            // keys per prompt-attention tile
#ifndef POP_GEMV_WAVES
#define POP_GEMV_WAVES 2048
#endif
constexpr int kGemvTarget = POP_GEMV_WAVES;  // waves a decode projection aims for
#ifndef POP_GEMV_INFLIGHT
#define POP_GEMV_INFLIGHT 16
#endif
constexpr int kGemvInflight = POP_GEMV_INFLIGHT;  // row loads in flight per lane
constexpr int kSumLanes = 16;                // lanes that share one output's chunk sum
#ifndef POP_LAYER_GEMM_BATCH
// bf16 decode batches from this size take both projections on the matrix cores (k_gemm_decode): the
// scalar GEMV's time grows with the batch (16 FMAs per weight element at batch 16: 60 us for q|k|v), the
// matrix-core kernel's stays near its weight stream (33 us at batch 16)
#define POP_LAYER_GEMM_BATCH 12
#endif
constexpr int kGdLanes = 8;  // lanes per output that add up k_gemm_decode's reduction slices
#ifndef POP_GEMV_PART_DIV
#define POP_GEMV_PART_DIV 8  // partial sums kept under (weight bytes) * 4 / POP_GEMV_PART_DIV
#endif
#ifndef POP_GEMV_WPB
#define POP_GEMV_WPB 1
#endif
constexpr int kGemvWaves = POP_GEMV_WPB;     // waves per block, on adjacent column groups of the same rows
constexpr int kLayerMaxBatch = 64;  // decode rows per layer call

__device__ __forceinline__ float elem_f(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float elem_f(const bf16s* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i].bits << 16);
}
// fp32 -> dtype, bf16 by round to nearest, ties to even (finite inputs).
__device__ __forceinline__ void put_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void put_elem(bf16s* p, int64_t i, float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7fffu + ((b >> 16) & 1u);
  p[i].bits = (uint16_t)(b >> 16);
}

// ---------------------------------------------------------------- RMSNorm
// out[row] = x[row] / sqrt(mean(x[row]^2) + eps) * g, one 256-thread block per
// row; the squares are summed per thread (ascending float4 slots), then per
// wave and across the four waves in order.  D % 4 == 0.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, int D, const float* __restrict__ g,
                                                 float eps, T* __restrict__ out) {
  __shared__ float wsum[4];
  const int64_t row = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + row * D);
  float s = 0.f;
  for (int i = threadIdx.x; i < D / 4; i += 256) {
    const float4 v = xr[i];
    s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  const float ms = (((wsum[0] + wsum[1]) + wsum[2]) + wsum[3]) / (float)D;
  const float inv = 1.0f / sqrtf(ms + eps);
  for (int i = threadIdx.x; i < D / 4; i += 256) {
    const float4 v = xr[i];
    const int64_t o = row * D + 4 * i;
    put_elem(out, o + 0, v.x * inv * g[4 * i + 0]);
    put_elem(out, o + 1, v.y * inv * g[4 * i + 1]);
    put_elem(out, o + 2, v.z * inv * g[4 * i + 2]);
    put_elem(out, o + 3, v.w * inv * g[4 * i + 3]);
  }
}

// ---------------------------------------------------------------- decode projections
// The projection's input x[b][k], by mode:
//   kXPlain  x in the dtype, [B, K];
//   kXNorm   RMSNorm of the fp32 residual stream res [B, K] with gain g,
//            rounded to the dtype as a stored RMSNorm output would be: each
//            wave first sums res[b]^2 itself (lane l over the float4 slots
//            l, l + 64, ..., then a butterfly: every wave gets the same bits);
//   kXCombine the attention output: the log-sum-exp merge of the 64-key slices
//            (ml [B, H, S, 2], po [B, H, S, hd]) for row k = head * hd + d,
//            rounded to the dtype; lane u of the wave merges row r0 + u of its
//            chunk (rows_per_chunk <= 64) and the values are broadcast by lane.
constexpr int kXPlain = 0, kXNorm = 1, kXCombine = 2;

struct GemvIn {
  const void* x;       // kXPlain
  const float* res;    // kXNorm
  const float* gain;
  float eps;
  const float* ml;     // kXCombine
  const float* po;
  int slices, hd, H;
};

template <typename T>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (sizeof(T) == 2) {
    uint32_t b = __float_as_uint(v);
    b += 0x7fffu + ((b >> 16) & 1u);
    return __uint_as_float((b >> 16) << 16);
  } else {
    return v;
  }
}

// Merged attention output of (sequence b, row k = head * hd + d): the slices
// in order, each rescaled by exp(m_s - max m) (log-sum-exp merge).
__device__ __forceinline__ float combine_row(const float* __restrict__ ml, const float* __restrict__ po, int S,
                                             int hd, int H, int b, int k) {
  const int h = k / hd, d = k % hd;
  const int64_t base = ((int64_t)b * H + h) * S;
  float M = -INFINITY;
#pragma unroll 4
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * (base + s)]);
  float l = 0.f, o = 0.f;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float e = expf(ml[2 * (base + s)] - M);
    l = fmaf(ml[2 * (base + s) + 1], e, l);
    o = fmaf(po[(base + s) * hd + d], e, o);
  }
  return o / l;
}

// part[chunk][b][n] = sum over rows k of the chunk of x[b][k] W[k][n].
// One wave per block: lane l owns columns n0 + V*l .. + V (one 16-byte load
// per row); the wave streams rows_per_chunk rows, kGemvInflight loads in
// flight, for BT tokens (blockIdx.z picks the token group).  Rows past the
// chunk are clamped for the load and their x taken as 0; token slots past B
// read row B - 1 and are not written.  N % V == 0; a lane whose columns lie
// past N loads the last vector and writes nothing.
template <typename T, int BT, int XM>
__global__ __launch_bounds__(64 * kGemvWaves) void k_gemv_kmajor(GemvIn in, int B, int K, const T* __restrict__ W,
                                                                 int N, int rows_per_chunk, float* __restrict__ part) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int n0 = ((blockIdx.x * kGemvWaves + (int)(threadIdx.x >> 6)) * 64 + lane) * V;
  const int nc = min(n0, N - V);
  const int chunk = blockIdx.y;
  const int b0 = blockIdx.z * BT;
  const int r0 = chunk * rows_per_chunk;
  const int r1 = min(r0 + rows_per_chunk, K);
  u32x4 w[kGemvInflight];
#pragma unroll
  for (int u = 0; u < kGemvInflight; ++u) w[u] = ld16_stream(W + (int64_t)min(r0 + u, r1 - 1) * N + nc);
  float inv[BT];    // kXNorm: 1 / rms of each token's residual row
  float mine[BT];   // kXCombine: the merged value of row r0 + lane
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    const int b = min(b0 + t, B - 1);
    inv[t] = 0.f;
    mine[t] = 0.f;
    if constexpr (XM == kXNorm) {
      const float4* xr = reinterpret_cast<const float4*>(in.res + (int64_t)b * K);
      float q = 0.f;
      for (int i = lane; i < K / 4; i += 64) {
        const float4 v = xr[i];
        q += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      q = wave_sum(q);
      inv[t] = 1.0f / sqrtf(q / (float)K + in.eps);
    }
    if constexpr (XM == kXCombine) {
      if (r0 + lane < r1) mine[t] = round_to<T>(combine_row(in.ml, in.po, in.slices, in.hd, in.H, b, r0 + lane));
    }
  }
  auto xval = [&](int t, int row) -> float {
    const int b = min(b0 + t, B - 1);
    if constexpr (XM == kXPlain) {
      return elem_f((const T*)in.x, (int64_t)b * K + row);
    } else if constexpr (XM == kXNorm) {
      return round_to<T>(in.res[(int64_t)b * K + row] * inv[t] * in.gain[row]);
    } else {
      return __shfl(mine[t], row - r0);
    }
  };
  float acc[BT][V];
#pragma unroll
  for (int t = 0; t < BT; ++t)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[t][v] = 0.f;
  for (int r = r0; r < r1; r += kGemvInflight) {
    if (r != r0) {
#pragma unroll
      for (int u = 0; u < kGemvInflight; ++u) w[u] = ld16_stream(W + (int64_t)min(r + u, r1 - 1) * N + nc);
    }
#pragma unroll
    for (int u = 0; u < kGemvInflight; ++u) {
      float wf[V];
      unpack(w[u], wf, T{});
      const bool ok = r + u < r1;
      const int row = min(r + u, r1 - 1);
#pragma unroll
      for (int t = 0; t < BT; ++t) {
        const float xv = xval(t, row);
        const float xs = ok ? xv : 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) acc[t][v] = fmaf(xs, wf[v], acc[t][v]);
      }
    }
  }
  if (n0 >= N) return;
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    if (b0 + t < B) {
      float* o = part + ((int64_t)chunk * B + b0 + t) * N + n0;
#pragma unroll
      for (int v = 0; v < V; v += 4) {
        // (non-temporal stores here measured slower: the next kernel then misses in L2)
        *reinterpret_cast<float4*>(o + v) = make_float4(acc[t][v], acc[t][v + 1], acc[t][v + 2], acc[t][v + 3]);
      }
    }
  }
}

// ---------------------------------------------------------------- q, k, v
// G lanes per (row m, column pair 2p, 2p+1) of q|k|v, rows outermost: lane j
// of the group adds chunks j, j + G, ... (ascending), and a butterfly over the
// G lanes (fp addition commutes, so every lane ends with the same bits) gives
// the pair's sums; then for q and k the rotation of the pair by
// pos * theta^(-2i/hd) (i = pair index inside the head; the angle, its sine
// and cosine in double precision).  Row m is token m % rows_per_seq of
// sequence m / rows_per_seq, at position pos0 + (*pos_ptr if given) +
// m % rows_per_seq.  q goes to q_out [M, H, hd] (fp32); k and v to the caches
// [seq, H_kv, L, hd] (dtype) when 0 <= pos < L, else nowhere.
template <typename T, int G>
__global__ __launch_bounds__(256) void k_qkv_rope(const float* __restrict__ part, int chunks, int M, int H, int Hkv,
                                                  int hd, int rows_per_seq, int pos0, const int32_t* __restrict__ pos_ptr,
                                                  double theta, int L, float* __restrict__ q_out, T* __restrict__ Kc,
                                                  T* __restrict__ Vc) {
  const int Nqkv = (H + 2 * Hkv) * hd;
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / G;
  const int j = threadIdx.x % G;
  if (t >= (int64_t)M * (Nqkv / 2)) return;  // whole groups leave together (256 % G == 0)
  const int m = (int)(t / (Nqkv / 2));
  const int col = 2 * (int)(t % (Nqkv / 2));
  float a = 0.f, b = 0.f;
  for (int c = j; c < chunks; c += G) {
    const float2 v = *reinterpret_cast<const float2*>(part + ((int64_t)c * M + m) * Nqkv + col);
    a += v.x;
    b += v.y;
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  if (j != 0) return;
  const int seq = m / rows_per_seq;
  const int pos = pos0 + (pos_ptr != nullptr ? *pos_ptr : 0) + m % rows_per_seq;
  const int head = col / hd, dd = col % hd;
  if (head < H + Hkv) {
    const double ang = (double)pos * pow(theta, -(double)dd / (double)hd);  // dd = 2i
    double sn, cs;
    sincos(ang, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float ra = a * c - b * s, rb = a * s + b * c;
    a = ra;
    b = rb;
  }
  if (head < H) {
    float* q = q_out + ((int64_t)m * H + head) * hd + dd;
    q[0] = a;
    q[1] = b;
    return;
  }
  if (pos < 0 || pos >= L) return;
  const int kvh = head < H + Hkv ? head - H : head - H - Hkv;
  T* dst = (head < H + Hkv ? Kc : Vc) + (((int64_t)seq * Hkv + kvh) * L + pos) * hd + dd;
  put_elem(dst, 0, a);
  put_elem(dst, 1, b);
}

// ---------------------------------------------------------------- decode attention
// Block (slice s, head h, sequence b): keys [s * 64, min(s * 64 + 64, n)) of
// the cache, n = pos + 1.  LPK = HD / V lanes share one key row (16-byte
// loads); 256 / LPK keys per pass.  The scores (q pre-scaled by 1/sqrt(hd))
// go to LDS; the slice max, the weights p = exp(s - max) and their sum follow;
// each thread adds its keys' p * v for its V dimensions, and the 256 / LPK key
// groups are summed in order.  Output per slice: (max, sum) and the
// unnormalised output [hd]; an empty slice writes (-inf, 0) and zeros.
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_decode(const float* __restrict__ q, const T* __restrict__ Kc,
                                                     const T* __restrict__ Vc, int L, int H, int Hkv,
                                                     const int32_t* __restrict__ pos_ptr, int n_slices,
                                                     float* __restrict__ part_ml, float* __restrict__ part_o) {
  constexpr int V = Vec<T>::N;
  constexpr int LPK = HD / V;
  constexpr int KPP = 256 / LPK;
  constexpr int PASSES = kAttnKeys / KPP;
  static_assert(LPK <= 64 && (LPK & (LPK - 1)) == 0 && PASSES >= 1, "head size");
  __shared__ float sc[kAttnKeys];
  __shared__ float red[KPP][HD + 1];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, c = tid % LPK, jj = tid / LPK;
  const int pos = *pos_ptr;
  const int n_keys = (pos >= 0 && pos < L) ? pos + 1 : 0;
  const int k0 = s * kAttnKeys, k1 = min(k0 + kAttnKeys, n_keys);
  const int64_t slot = ((int64_t)b * H + h) * n_slices + s;
  if (k0 >= k1) {
    if (tid == 0) {
      part_ml[2 * slot] = -INFINITY;
      part_ml[2 * slot + 1] = 0.f;
    }
    if (tid < HD) part_o[slot * HD + tid] = 0.f;
    return;
  }
  const int kvh = h / (H / Hkv);
  const T* Kb = Kc + ((int64_t)b * Hkv + kvh) * L * HD;
  const T* Vb = Vc + ((int64_t)b * Hkv + kvh) * L * HD;
  const float scale = 1.0f / sqrtf((float)HD);
  float qf[V];
#pragma unroll
  for (int v = 0; v < V; ++v) qf[v] = q[((int64_t)b * H + h) * HD + c * V + v] * scale;
  u32x4 kr[PASSES], vr[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int key = min(k0 + jj + p * KPP, k1 - 1);
    kr[p] = ld16(Kb + (int64_t)key * HD + c * V);
    vr[p] = ld16(Vb + (int64_t)key * HD + c * V);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float kf[V];
    unpack(kr[p], kf, T{});
    float d = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) d = fmaf(qf[v], kf[v], d);
#pragma unroll
    for (int o = LPK / 2; o > 0; o >>= 1) d += __shfl_xor(d, o);
    const int j = jj + p * KPP;
    if (c == 0) sc[j] = k0 + j < k1 ? d : -INFINITY;
  }
  __syncthreads();
  float mx = -INFINITY;
#pragma unroll 8
  for (int j = 0; j < kAttnKeys; ++j) mx = fmaxf(mx, sc[j]);
  __syncthreads();
  if (tid < kAttnKeys) sc[tid] = expf(sc[tid] - mx);  // masked keys: exp(-inf) = 0
  __syncthreads();
  float o[V];
#pragma unroll
  for (int v = 0; v < V; ++v) o[v] = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const float w = sc[jj + p * KPP];
    float vf[V];
    unpack(vr[p], vf, T{});
#pragma unroll
    for (int v = 0; v < V; ++v) o[v] = fmaf(w, vf[v], o[v]);
  }
#pragma unroll
  for (int v = 0; v < V; ++v) red[jj][c * V + v] = o[v];
  __syncthreads();
  if (tid < HD) {
    float a = 0.f;
    for (int g = 0; g < KPP; ++g) a += red[g][tid];
    part_o[slot * HD + tid] = a;
  }
  if (tid == 0) {
    float l = 0.f;
    for (int j = 0; j < kAttnKeys; ++j) l += sc[j];
    part_ml[2 * slot] = mx;
    part_ml[2 * slot + 1] = l;
  }
}

// The slices' merge as a kernel of its own (batches above 2, where merging
// inside every wave of the output projection would repeat it per token):
// out[b, h*hd + d] = combine_row(b, h*hd + d), rounded to the dtype; one block
// of hd threads per (head, sequence).
template <typename T>
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ ml, const float* __restrict__ po, int S,
                                                    int H, int hd, T* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  if (d >= hd) return;
  put_elem(out, ((int64_t)b * H + h) * hd + d, combine_row(ml, po, S, hd, H, b, h * hd + d));
}

// ---------------------------------------------------------------- prompt attention
// Block (query tile qt, head h, sequence b): queries q0 .. q0 + 15 (q0 = 16 qt)
// of the sequence's N prompt tokens, keys 0 .. q0 + 15 in 32-key tiles staged
// in LDS as fp32.  Thread (row r = tid / 16, u = tid % 16) scores keys u and
// u + 16 of the tile for query r, keeps the row's running max and sum (the 16
// lanes of a row agree: the reductions are butterflies over them), and owns
// output dimensions u + 16 i.  Keys after the query are masked; rows past N
// compute on zeros and are not written.
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_prefill(const float* __restrict__ q, const T* __restrict__ Kc,
                                                      const T* __restrict__ Vc, int N, int L, int H, int Hkv,
                                                      T* __restrict__ out) {
  constexpr int DI = HD / 16;
  __shared__ float Qs[kPfQ][HD];
  __shared__ float Ks[kPfK][HD + 1];
  __shared__ float Vs[kPfK][HD];
  __shared__ float Ps[kPfQ][kPfK + 1];
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, r = tid / 16, u = tid % 16;
  const int q0 = qt * kPfQ;
  const int kvh = h / (H / Hkv);
  const T* Kb = Kc + ((int64_t)b * Hkv + kvh) * L * HD;
  const T* Vb = Vc + ((int64_t)b * Hkv + kvh) * L * HD;
  const float scale = 1.0f / sqrtf((float)HD);
  for (int i = tid; i < kPfQ * HD; i += 256) {
    const int rr = i / HD, dd = i % HD;
    Qs[rr][dd] = q0 + rr < N ? q[(((int64_t)b * N + q0 + rr) * H + h) * HD + dd] * scale : 0.f;
  }
  const int qpos = q0 + r;                       // this row's position
  const int kend = min(q0 + kPfQ, N);            // keys the tile's last query sees
  float m_run = -INFINITY, l_run = 0.f, o[DI];
#pragma unroll
  for (int i = 0; i < DI; ++i) o[i] = 0.f;
  for (int t0 = 0; t0 < kend; t0 += kPfK) {
    __syncthreads();
    for (int i = tid; i < kPfK * HD; i += 256) {
      const int j = i / HD, dd = i % HD;
      const int key = min(t0 + j, kend - 1);
      Ks[j][dd] = elem_f(Kb, (int64_t)key * HD + dd);
      Vs[j][dd] = elem_f(Vb, (int64_t)key * HD + dd);
    }
    __syncthreads();
    float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
    for (int dd = 0; dd < HD; ++dd) {
      const float qv = Qs[r][dd];
      s0 = fmaf(qv, Ks[u][dd], s0);
      s1 = fmaf(qv, Ks[u + 16][dd], s1);
    }
    const bool row_ok = qpos < N;
    if (t0 + u > qpos) s0 = row_ok ? -INFINITY : 0.f;
    if (t0 + u + 16 > qpos) s1 = row_ok ? -INFINITY : 0.f;
    float mt = fmaxf(s0, s1);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
    const float m_new = fmaxf(m_run, mt);  // finite: key 0 is in every row's window
    const float corr = expf(m_run - m_new);
    const float p0 = expf(s0 - m_new), p1 = expf(s1 - m_new);
    float ps = p0 + p1;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    l_run = l_run * corr + ps;
    m_run = m_new;
    Ps[r][u] = p0;
    Ps[r][u + 16] = p1;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DI; ++i) {
      float a = o[i] * corr;
      const int dd = u + 16 * i;
#pragma unroll 8
      for (int j = 0; j < kPfK; ++j) a = fmaf(Ps[r][j], Vs[j][dd], a);
      o[i] = a;
    }
  }
  if (qpos >= N) return;
  T* dst = out + (((int64_t)b * N + qpos) * H + h) * HD;
#pragma unroll
  for (int i = 0; i < DI; ++i) put_elem(dst, u + 16 * i, o[i] / l_run);
}

// ---------------------------------------------------------------- prompt attention, matrix cores
// bf16: S = Q K^T and O += P V on v_mfma_f32_16x16x32_bf16.  Block (query tile
// of 64, head h, sequence b); wave w owns queries q0 + 16 w + [0, 16).  Per
// 64-key tile of the causal window: K staged in LDS key-major (the B operand of
// Q K^T reads 8 consecutive dims of one key), V staged transposed (the B
// operand of P V reads 8 consecutive keys of one dim), both with padded pitches.
// The fp32 operands q and P enter as two bf16 parts each, hi = bf16(v) and
// lo = bf16(v - hi), and both parts are multiplied (about 16 significant bits,
// so the products carry fp32-level error, not bf16 rounding of q and P); K
// and V are bf16 already.  The scores are scaled by 1/sqrt(hd) in fp32.
// Online softmax on the accumulators: lane l holds rows 4 (l >> 4) + e,
// columns l & 15 of each 16 x 16 tile, so a row's max and sum are butterflies
// over the 16 lanes sharing l >> 4.  P's parts go to the wave's LDS slices and
// are read back as A operands.  Query rows past N load row N - 1 and are not
// written.
constexpr int kMq = 64, kMk = 64;

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

template <int HD>
__global__ __launch_bounds__(256) void k_attn_prefill_mfma(const float* __restrict__ q, const bf16s* __restrict__ Kc,
                                                           const bf16s* __restrict__ Vc, int N, int L, int H, int Hkv,
                                                           bf16s* __restrict__ out) {
  constexpr int KP = HD + 8;    // Ks pitch (bf16)
  constexpr int VP = kMk + 8;   // Vt and Ps pitch (bf16)
  constexpr int KS = HD / 32;   // k-steps of Q K^T
  constexpr int DT = HD / 16;   // 16-dim output tiles
  __shared__ __align__(16) uint16_t Ks[kMk * KP];
  __shared__ __align__(16) uint16_t Vt[HD * VP];
  __shared__ __align__(16) uint16_t Ps[4][2][16 * VP];  // per wave: P's hi and lo parts
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = qt * kMq;
  const int kvh = h / (H / Hkv);
  const bf16s* Kb = Kc + ((int64_t)b * Hkv + kvh) * L * HD;
  const bf16s* Vb = Vc + ((int64_t)b * Hkv + kvh) * L * HD;
  const int fr = lane & 15, fg = lane >> 4;
  // Q fragments: row q0 + 16 wave + fr, dims 8 fg + 32 ks
  bf16x8_t qa[KS], qb[KS];  // q's hi and lo parts
  {
    const int row = min(q0 + 16 * wave + fr, N - 1);
    const float* qr = q + (((int64_t)b * N + row) * H + h) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 a = *reinterpret_cast<const float4*>(qr + 32 * ks + 8 * fg);
      const float4 c = *reinterpret_cast<const float4*>(qr + 32 * ks + 8 * fg + 4);
      const float f[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      u32x4 uh, ul;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t h0 = bf16_bits_rne(f[2 * x]), h1 = bf16_bits_rne(f[2 * x + 1]);
        const uint32_t l0 = bf16_bits_rne(f[2 * x] - __uint_as_float(h0 << 16));
        const uint32_t l1 = bf16_bits_rne(f[2 * x + 1] - __uint_as_float(h1 << 16));
        uh[x] = h0 | (h1 << 16);
        ul[x] = l0 | (l1 << 16);
      }
      qa[ks] = __builtin_bit_cast(bf16x8_t, uh);
      qb[ks] = __builtin_bit_cast(bf16x8_t, ul);
    }
  }
  const float scale = 1.0f / sqrtf((float)HD);
  float m_run[4], l_run[4];
  f32x4_t acc_o[DT];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m_run[e] = -INFINITY;
    l_run[e] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < DT; ++t) acc_o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kend = min(q0 + kMq, N);
  for (int t0 = 0; t0 < kend; t0 += kMk) {
    __syncthreads();
    // K tile: row j = key t0 + j (clamped), 16-byte pieces
    for (int i = tid; i < kMk * HD / 8; i += 256) {
      const int j = i / (HD / 8), c = (i % (HD / 8)) * 8;
      const int key = min(t0 + j, kend - 1);
      *reinterpret_cast<u32x4*>(&Ks[j * KP + c]) = ld16(Kb + (int64_t)key * HD + c);
    }
    // V tile transposed: a thread takes keys 2p, 2p + 1 and dims c .. c + 7
    for (int i = tid; i < (kMk / 2) * (HD / 8); i += 256) {
      const int pr = i / (HD / 8), c = (i % (HD / 8)) * 8;
      const int k0 = min(t0 + 2 * pr, kend - 1), k1 = min(t0 + 2 * pr + 1, kend - 1);
      const u32x4 v0 = ld16(Vb + (int64_t)k0 * HD + c), v1 = ld16(Vb + (int64_t)k1 * HD + c);
      uint32_t* vt32 = reinterpret_cast<uint32_t*>(Vt);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t lo = (v0[x >> 1] >> ((x & 1) * 16)) & 0xffffu;
        const uint32_t hi = (v1[x >> 1] >> ((x & 1) * 16)) & 0xffffu;
        vt32[((c + x) * VP) / 2 + pr] = lo | (hi << 16);
      }
    }
    __syncthreads();
    // S = Q K^T for 4 tiles of 16 keys
    f32x4_t sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t kb = *reinterpret_cast<const bf16x8_t*>(&Ks[(16 * j + fr) * KP + 32 * ks + 8 * fg]);
        sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, sc[j], 0, 0, 0);
        sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[ks], kb, sc[j], 0, 0, 0);
      }
    }
    // mask, scale, online softmax per row (rows 4 fg + e of the wave's 16)
    float corr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qrow = q0 + 16 * wave + 4 * fg + e;
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = t0 + 16 * j + fr;
        float v = sc[j][e] * scale;
        if (key > qrow) v = qrow < N ? -INFINITY : 0.f;  // causal mask; padding rows stay finite
        sc[j][e] = v;
        mt = fmaxf(mt, v);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
      const float m_new = fmaxf(m_run[e], mt);  // finite: key 0 is in every row's window
      corr[e] = expf(m_run[e] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = expf(sc[j][e] - m_new);
        sc[j][e] = pv;
        ps += pv;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o);
      l_run[e] = l_run[e] * corr[e] + ps;
      m_run[e] = m_new;
    }
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc_o[t][e] *= corr[e];
    // P's two bf16 parts to this wave's LDS slices: row 4 fg + e, key 16 j + fr
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t hp = bf16_bits_rne(sc[j][e]);
        Ps[wave][0][(4 * fg + e) * VP + 16 * j + fr] = (uint16_t)hp;
        Ps[wave][1][(4 * fg + e) * VP + 16 * j + fr] = (uint16_t)bf16_bits_rne(sc[j][e] - __uint_as_float(hp << 16));
      }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes land before its reads
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    // O += P V: 2 k-steps of 32 keys per 16-dim tile
#pragma unroll
    for (int kk = 0; kk < kMk / 32; ++kk) {
      const bf16x8_t pa = *reinterpret_cast<const bf16x8_t*>(&Ps[wave][0][fr * VP + 32 * kk + 8 * fg]);
      const bf16x8_t pb = *reinterpret_cast<const bf16x8_t*>(&Ps[wave][1][fr * VP + 32 * kk + 8 * fg]);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8_t vb = *reinterpret_cast<const bf16x8_t*>(&Vt[(16 * t + fr) * VP + 32 * kk + 8 * fg]);
        acc_o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc_o[t], 0, 0, 0);
        acc_o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, vb, acc_o[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int qrow = q0 + 16 * wave + 4 * fg + e;
    if (qrow >= N) continue;
    bf16s* dst = out + (((int64_t)b * N + qrow) * H + h) * HD;
    const float inv = 1.0f / l_run[e];
#pragma unroll
    for (int t = 0; t < DT; ++t) dst[16 * t + fr].bits = (uint16_t)bf16_bits_rne(acc_o[t][e] * inv);
  }
}

// ---------------------------------------------------------------- decode projections, matrix cores
// bf16, 12 or more tokens: part[slice][b][n] = sum over rows k of the slice of
// x[b][k] W[k][n] on v_mfma_f32_16x16x32_bf16.  Block (256-column tile, slice
// of the reduction, group of 16 tokens); wave w owns columns 64 w + [0, 64) of
// the tile (four 16-column MFMA tiles).  A stage is 32 rows x 256 columns of W
// (512 contiguous bytes per row): loaded to registers one stage ahead, written
// to LDS transposed (two rows packed per 32-bit word, so a column's 8
// consecutive k are one 16-byte read: the B operand), two LDS buffers.  The A
// operand (16 tokens x 32 k of x) is read from global memory (small, cached);
// token slots past B read token B - 1 and are not written; columns past N read
// the last vector and are not written.  K-range and slice length are
// multiples of 32.
constexpr int kGdBN = 256, kGdBK = 32, kGdKP = kGdBK + 8;

__global__ __launch_bounds__(256) void k_gemm_decode(const bf16s* __restrict__ x, int B, int K,
                                                     const bf16s* __restrict__ W, int N, int kslice,
                                                     float* __restrict__ part) {
  __shared__ __align__(16) uint16_t Bt[2][kGdBN * kGdKP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * kGdBN, sl = blockIdx.y, b0 = blockIdx.z * 16;
  const int k0 = sl * kslice, k1 = min(k0 + kslice, K);
  const int ns = (k1 - k0) / kGdBK;
  // staging units: (row pair p, 8-column group g); 16 x 32 units, two per thread;
  // consecutive threads take consecutive row pairs, so their packed LDS words are
  // consecutive (the 16 lanes of a column group hit 16 banks)
  u32x4 r0[2], r1[2];
  auto fetch = [&](int st) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int unit = tid + 256 * u, p = unit & 15, g = unit >> 4;
      const int col = min(n0 + 8 * g, N - 8);
      const int64_t row = k0 + st * kGdBK + 2 * p;
      r0[u] = ld16_stream(W + row * N + col);
      r1[u] = ld16_stream(W + (row + 1) * N + col);
    }
  };
  auto stash = [&](int buf) {
    uint32_t* b32 = reinterpret_cast<uint32_t*>(Bt[buf]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int unit = tid + 256 * u, p = unit & 15, g = unit >> 4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (r0[u][j >> 1] >> ((j & 1) * 16)) & 0xffffu;
        const uint32_t hi = (r1[u][j >> 1] >> ((j & 1) * 16)) & 0xffffu;
        b32[((8 * g + j) * kGdKP) / 2 + p] = lo | (hi << 16);
      }
    }
  };
  const int fr = lane & 15, fg = lane >> 4;
  const bf16s* xr = x + (int64_t)min(b0 + fr, B - 1) * K + 8 * fg;
  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  stash(0);
  __syncthreads();
  for (int st = 0; st < ns; ++st) {
    if (st + 1 < ns) fetch(st + 1);
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ld16(xr + k0 + st * kGdBK));
    const uint16_t* bt = Bt[st & 1];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&bt[(64 * wave + 16 * t + fr) * kGdKP + 8 * fg]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[t], 0, 0, 0);
    }
    if (st + 1 < ns) stash((st + 1) & 1);
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int col = n0 + 64 * wave + 16 * t + fr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = b0 + 4 * fg + e;
      if (b < B && col < N) part[((int64_t)sl * B + b) * N + col] = acc[t][e];
    }
  }
}

// ---------------------------------------------------------------- residual
// x[i] += sum over chunks of part[c][i]: G lanes per output, lane j adding
// chunks j, j + G, ... in order, then a butterfly over the G lanes.
template <int G>
__global__ __launch_bounds__(256) void k_sum_residual(const float* __restrict__ part, int chunks, int64_t n,
                                                      float* __restrict__ x) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) / G;
  const int j = threadIdx.x % G;
  if (i >= n) return;  // whole groups leave together
  float s = 0.f;
  for (int c = j; c < chunks; c += G) s += part[c * n + i];
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (j == 0) x[i] += s;
}

__global__ __launch_bounds__(256) void k_add(float* __restrict__ x, const float* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] += y[i];
}

// ---------------------------------------------------------------- host
struct GemvPlan {
  int bt, groups, rows_per_chunk, chunks, col_blocks;
};

// Rows per chunk: enough waves to fill the chip, but the partial sums kept
// under an eighth of the weight bytes (they are written and read once more).
static GemvPlan gemv_plan(int B, int K, int N, int esz, int max_rows = 0) {
  GemvPlan p;
  p.bt = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16;
  p.groups = (B + p.bt - 1) / p.bt;
  const int V = 16 / esz;
  p.col_blocks = (N + 64 * V - 1) / (64 * V);
  int want = (kGemvTarget + p.col_blocks * p.groups - 1) / (p.col_blocks * p.groups);
  const int64_t cap = ((int64_t)K * esz) / (POP_GEMV_PART_DIV * (int64_t)(B > 0 ? B : 1));
  if (want > cap) want = (int)(cap > 1 ? cap : 1);
  if (want < 1) want = 1;
  int rpc = (K + want - 1) / want;
  rpc = (rpc + kGemvInflight - 1) / kGemvInflight * kGemvInflight;
  if (max_rows > 0 && rpc > max_rows) rpc = max_rows;
  p.rows_per_chunk = rpc;
  p.chunks = (K + rpc - 1) / rpc;
  return p;
}

template <typename T, int XM>
static void launch_gemv(hipStream_t st, const GemvPlan& p, const GemvIn& in, int B, int K, const void* W, int N,
                        float* part) {
  const dim3 grid((p.col_blocks + kGemvWaves - 1) / kGemvWaves, p.chunks, p.groups);
  const dim3 blk(64 * kGemvWaves);
  const T* ww = (const T*)W;
  switch (p.bt) {
    case 1: POP_LAUNCH((k_gemv_kmajor<T, 1, XM>), grid, blk, 0, st, in, B, K, ww, N, p.rows_per_chunk, part); break;
    case 2: POP_LAUNCH((k_gemv_kmajor<T, 2, XM>), grid, blk, 0, st, in, B, K, ww, N, p.rows_per_chunk, part); break;
    case 4: POP_LAUNCH((k_gemv_kmajor<T, 4, XM>), grid, blk, 0, st, in, B, K, ww, N, p.rows_per_chunk, part); break;
    case 8: POP_LAUNCH((k_gemv_kmajor<T, 8, XM>), grid, blk, 0, st, in, B, K, ww, N, p.rows_per_chunk, part); break;
    default: POP_LAUNCH((k_gemv_kmajor<T, 16, XM>), grid, blk, 0, st, in, B, K, ww, N, p.rows_per_chunk, part); break;
  }
}

// Slices of the reduction for k_gemm_decode: enough blocks to fill the chip.
static int gd_kslice(int B, int K, int N) {
  const int blocks = ((N + kGdBN - 1) / kGdBN) * ((B + 15) / 16);
  int want = (512 + blocks - 1) / blocks;  // (partial sums stay a fraction of the weight bytes)
  if (want > K / kGdBK) want = K / kGdBK;
  if (want < 1) want = 1;
  return (K / want + kGdBK - 1) / kGdBK * kGdBK;
}
static int gd_slices(int B, int K, int N) {
  const int ks = gd_kslice(B, K, N);
  return (K + ks - 1) / ks;
}
static int launch_gemm_decode(hipStream_t st, const void* x, int B, int K, const void* W, int N, float* part) {
  const int ks = gd_kslice(B, K, N), ns = (K + ks - 1) / ks;
  POP_LAUNCH(k_gemm_decode, dim3((N + kGdBN - 1) / kGdBN, ns, (B + 15) / 16), dim3(256), 0, st, (const bf16s*)x, B,
             K, (const bf16s*)W, N, ks, part);
  return ns;
}

static int n_qkv(const pop_layer_shape& s) { return (s.n_heads + 2 * s.n_kv_heads) * s.head_dim; }
static int n_slices(const pop_layer_shape& s) { return (s.cache_len + kAttnKeys - 1) / kAttnKeys; }
static dim3 qkv_grid(int64_t M, const pop_layer_shape& s, int G) {
  return dim3((unsigned)((M * (n_qkv(s) / 2) * G + 255) / 256));
}

static pop_status check_layer(const pop_layer_shape* s, pop_dtype dt) {
  if (s == nullptr) return fail(POP_ERR_INVALID_ARGUMENT, "shape is NULL");
  pop_status st = check_dtype_width(dt, s->d);
  if (st != POP_OK) return st;
  if (s->d % 64 != 0) return fail(POP_ERR_BAD_SHAPE, "d=%d is not a multiple of 64", s->d);
  if (s->head_dim != 64 && s->head_dim != 128) return fail(POP_ERR_BAD_SHAPE, "head_dim=%d is not 64 or 128", s->head_dim);
  if (s->n_heads < 1 || s->n_kv_heads < 1 || s->n_heads % s->n_kv_heads != 0 || s->n_heads > 1024)
    return fail(POP_ERR_BAD_SHAPE, "n_heads=%d, n_kv_heads=%d: need 1 <= n_kv_heads, n_kv_heads | n_heads <= 1024",
                s->n_heads, s->n_kv_heads);
  if ((int64_t)(s->n_heads + 2 * s->n_kv_heads) * s->head_dim > 4 * POP_MAX_D)
    return fail(POP_ERR_BAD_SHAPE, "q|k|v width above %d", 4 * POP_MAX_D);
  if (s->d_ff < 1 || s->d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", s->d_ff, POP_MAX_D_FF);
  if (s->cache_len < 1 || s->cache_len > (1 << 20)) return fail(POP_ERR_BAD_SHAPE, "cache_len=%d outside [1, 2^20]", s->cache_len);
  if (!(s->eps >= 0.0) || !(s->rope_theta > 0.0)) return fail(POP_ERR_INVALID_ARGUMENT, "eps must be >= 0 and rope_theta > 0");
  return POP_OK;
}

static pop_status check_weights(const pop_layer_weights* w) {
  if (w == nullptr || w->attn_norm == nullptr || w->Wqkv_T == nullptr || w->Wo_T == nullptr || w->ffn_norm == nullptr ||
      w->W_gate == nullptr || w->W_up == nullptr || w->W_downT == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "a weight pointer is NULL");
  if (!aligned16(w->attn_norm) || !aligned16(w->Wqkv_T) || !aligned16(w->Wo_T) || !aligned16(w->ffn_norm) ||
      !aligned16(w->W_gate) || !aligned16(w->W_up) || !aligned16(w->W_downT))
    return fail(POP_ERR_MISALIGNED, "weights must be 16-byte aligned");
  return POP_OK;
}

struct DecodeLayerWs {
  char* xn;     // RMSNorm outputs, dtype [B, D] (the FFN's input after the call)
  float* part;  // projection partial sums
  float* q;     // [B, H, hd]
  float* ml;    // [B, H, slices, 2]
  float* po;    // [B, H, slices, hd]
  char* ao;     // merged attention output, dtype [B, H hd] (batches above 2)
  float* y;     // FFN output [B, D]
  char* ffn;    // FFN workspace
  size_t total;
};

static DecodeLayerWs decode_layer_ws(int B, const pop_layer_shape& s, pop_dtype dt, char* base) {
  const int e = elem_bytes(dt), Hd = s.n_heads * s.head_dim, S = n_slices(s);
  const GemvPlan a = gemv_plan(B, s.d, n_qkv(s), e), o = gemv_plan(B, Hd, s.d, e, 64);
  const int ks = std::max(gd_slices(B, s.d, n_qkv(s)), gd_slices(B, Hd, s.d));
  const size_t part =
      (size_t)std::max({(int64_t)a.chunks * n_qkv(s), (int64_t)o.chunks * s.d, (int64_t)ks * n_qkv(s),
                        (int64_t)ks * s.d}) * B * 4;
  DecodeLayerWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes > 0 ? bytes : 1, 256);
    return p;
  };
  w.xn = take((size_t)B * s.d * e);
  w.part = (float*)take(part);
  w.q = (float*)take((size_t)B * Hd * 4);
  w.ml = (float*)take((size_t)B * s.n_heads * S * 2 * 4);
  w.po = (float*)take((size_t)B * s.n_heads * S * s.head_dim * 4);
  w.ao = take((size_t)B * Hd * e);
  w.y = (float*)take((size_t)B * s.d * 4);
  w.ffn = take(pop_decode_workspace_bytes(B, s.d, s.d_ff));
  w.total = off;
  return w;
}

struct PrefillLayerWs {
  char* xn;  // dtype [M, D] (the FFN's input after the call)
  float* Y;  // [M, max(q|k|v width, D)]
  float* q;  // [M, H, hd]
  char* ao;  // dtype [M, H hd]
  char* ffn;
  size_t total;
};

static PrefillLayerWs prefill_layer_ws(int64_t M, const pop_layer_shape& s, pop_dtype dt, char* base) {
  const int e = elem_bytes(dt), Hd = s.n_heads * s.head_dim;
  PrefillLayerWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes > 0 ? bytes : 1, 256);
    return p;
  };
  w.xn = take((size_t)M * s.d * e);
  w.Y = (float*)take((size_t)M * std::max(n_qkv(s), s.d) * 4);
  w.q = (float*)take((size_t)M * Hd * 4);
  w.ao = take((size_t)M * Hd * e);
  w.ffn = take(pop_prefill_ffn_partition_workspace_bytes(M, s.d, s.d_ff, dt));
  w.total = off;
  return w;
}

template <typename T>
static void launch_attn_decode(hipStream_t st, const pop_layer_shape& s, int B, const void* Kc, const void* Vc,
                               const int32_t* pos, const DecodeLayerWs& w) {
  const int S = n_slices(s);
  const dim3 grid(S, s.n_heads, B);
  if (s.head_dim == 64)
    POP_LAUNCH((k_attn_decode<T, 64>), grid, dim3(256), 0, st, w.q, (const T*)Kc, (const T*)Vc, s.cache_len, s.n_heads,
               s.n_kv_heads, pos, S, w.ml, w.po);
  else
    POP_LAUNCH((k_attn_decode<T, 128>), grid, dim3(256), 0, st, w.q, (const T*)Kc, (const T*)Vc, s.cache_len, s.n_heads,
               s.n_kv_heads, pos, S, w.ml, w.po);
}

template <typename T>
static void launch_attn_prefill(hipStream_t st, const pop_layer_shape& s, int B, int N, const void* Kc, const void* Vc,
                                const PrefillLayerWs& w) {
  if constexpr (sizeof(T) == 2) {  // bf16: matrix cores
    const dim3 grid((N + kMq - 1) / kMq, s.n_heads, B);
    if (s.head_dim == 64)
      POP_LAUNCH((k_attn_prefill_mfma<64>), grid, dim3(256), 0, st, w.q, (const bf16s*)Kc, (const bf16s*)Vc, N,
                 s.cache_len, s.n_heads, s.n_kv_heads, (bf16s*)w.ao);
    else
      POP_LAUNCH((k_attn_prefill_mfma<128>), grid, dim3(256), 0, st, w.q, (const bf16s*)Kc, (const bf16s*)Vc, N,
                 s.cache_len, s.n_heads, s.n_kv_heads, (bf16s*)w.ao);
    return;
  }
  const dim3 grid((N + kPfQ - 1) / kPfQ, s.n_heads, B);
  if (s.head_dim == 64)
    POP_LAUNCH((k_attn_prefill<T, 64>), grid, dim3(256), 0, st, w.q, (const T*)Kc, (const T*)Vc, N, s.cache_len,
               s.n_heads, s.n_kv_heads, (T*)w.ao);
  else
    POP_LAUNCH((k_attn_prefill<T, 128>), grid, dim3(256), 0, st, w.q, (const T*)Kc, (const T*)Vc, N, s.cache_len,
               s.n_heads, s.n_kv_heads, (T*)w.ao);
}

// The attention half of a decode step, through the FFN's RMSNorm: x becomes h
// and lw.xn RMSNorm(h).  At batch <= 2 the attention RMSNorm runs inside the
// q|k|v projection and the slices' merge inside the output projection; above,
// each is a launch of its own.
template <typename T>
static void enqueue_layer_decode_attention(hipStream_t h, float* x, int batch, const pop_layer_shape& s,
                                           const pop_layer_weights* w, void* Kc, void* Vc, const int32_t* pos,
                                           const DecodeLayerWs& lw) {
  const int D = s.d, Hd = s.n_heads * s.head_dim, e = sizeof(T);
  const GemvPlan pq = gemv_plan(batch, D, n_qkv(s), e), po = gemv_plan(batch, Hd, D, e, 64);
  const bool fuse_norm = batch <= 2;
  // bf16 from POP_LAYER_GEMM_BATCH tokens: both projections on k_gemm_decode (matrix cores), in slices of
  // the reduction that the rotation and the residual sum add up
  const bool gemm_path = sizeof(T) == 2 && batch >= POP_LAYER_GEMM_BATCH;
  int qkv_slices = 1, o_slices = 1;  // partial products the matrix-core projections leave
  GemvIn qin{};
  if (fuse_norm) {
    qin.res = x;
    qin.gain = w->attn_norm;
    qin.eps = (float)s.eps;
    launch_gemv<T, kXNorm>(h, pq, qin, batch, D, w->Wqkv_T, n_qkv(s), lw.part);
  } else {
    POP_LAUNCH(k_rmsnorm<T>, dim3(batch), dim3(256), 0, h, x, D, w->attn_norm, (float)s.eps, (T*)lw.xn);
    qin.x = lw.xn;
    if (gemm_path)
      qkv_slices = launch_gemm_decode(h, lw.xn, batch, D, w->Wqkv_T, n_qkv(s), lw.part);
    else
      launch_gemv<T, kXPlain>(h, pq, qin, batch, D, w->Wqkv_T, n_qkv(s), lw.part);
  }
  if (gemm_path)
    POP_LAUNCH((k_qkv_rope<T, kGdLanes>), qkv_grid(batch, s, kGdLanes), dim3(256), 0, h, lw.part,
               qkv_slices, batch, s.n_heads, s.n_kv_heads, s.head_dim, 1, 0, pos, s.rope_theta,
               s.cache_len, lw.q, (T*)Kc, (T*)Vc);
  else
    POP_LAUNCH((k_qkv_rope<T, kSumLanes>), qkv_grid(batch, s, kSumLanes), dim3(256), 0, h, lw.part, pq.chunks, batch,
               s.n_heads, s.n_kv_heads, s.head_dim, 1, 0, pos, s.rope_theta, s.cache_len, lw.q, (T*)Kc, (T*)Vc);
  launch_attn_decode<T>(h, s, batch, Kc, Vc, pos, lw);
  GemvIn oin{};
  if (batch <= 2) {
    oin.ml = lw.ml;
    oin.po = lw.po;
    oin.slices = n_slices(s);
    oin.hd = s.head_dim;
    oin.H = s.n_heads;
    launch_gemv<T, kXCombine>(h, po, oin, batch, Hd, w->Wo_T, D, lw.part);
  } else {
    POP_LAUNCH(k_attn_merge<T>, dim3(s.n_heads, batch), dim3(128), 0, h, lw.ml, lw.po, n_slices(s), s.n_heads,
               s.head_dim, (T*)lw.ao);
    oin.x = lw.ao;
    if (gemm_path)
      o_slices = launch_gemm_decode(h, lw.ao, batch, Hd, w->Wo_T, D, lw.part);
    else
      launch_gemv<T, kXPlain>(h, po, oin, batch, Hd, w->Wo_T, D, lw.part);
  }
  // (A last-block-done fusion of the next two launches measured slower: every
  // block's device-scope release writes back its XCD's L2.)
  const int64_t n = (int64_t)batch * D;
  if (gemm_path)
    POP_LAUNCH(k_sum_residual<kGdLanes>, dim3((unsigned)((n * kGdLanes + 255) / 256)), dim3(256), 0, h,
               lw.part, o_slices, n, x);
  else
    POP_LAUNCH(k_sum_residual<kSumLanes>, dim3((unsigned)((n * kSumLanes + 255) / 256)), dim3(256), 0, h, lw.part,
               po.chunks, n, x);
  POP_LAUNCH(k_rmsnorm<T>, dim3(batch), dim3(256), 0, h, x, D, w->ffn_norm, (float)s.eps, (T*)lw.xn);
}

static pop_status launched_layer() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}

}  // namespace pop

using namespace pop;

extern "C" size_t pop_layer_decode_workspace_bytes(int32_t batch, const pop_layer_shape* s, pop_dtype dt) {
  clear_error();
  if (batch < 1 || batch > kLayerMaxBatch || check_layer(s, dt) != POP_OK) return 0;
  return decode_layer_ws(batch, *s, dt, nullptr).total;
}

extern "C" size_t pop_layer_prefill_workspace_bytes(int32_t batch, int32_t n_tokens, const pop_layer_shape* s,
                                                    pop_dtype dt) {
  clear_error();
  if (batch < 1 || n_tokens < 1 || check_layer(s, dt) != POP_OK || n_tokens > s->cache_len ||
      (int64_t)batch * n_tokens > (1 << 22))
    return 0;
  return prefill_layer_ws((int64_t)batch * n_tokens, *s, dt, nullptr).total;
}

extern "C" pop_status pop_layer_decode(float* x, int32_t batch, const pop_layer_shape* s, const pop_layer_weights* w,
                                       pop_dtype dt, void* K_cache, void* V_cache, const int32_t* pos,
                                       const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, double r,
                                       int32_t dense_ffn, int32_t* selected, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status st = check_layer(s, dt);
  if (st != POP_OK) return st;
  if ((st = check_weights(w)) != POP_OK) return st;
  if (batch < 1 || batch > kLayerMaxBatch) return fail(POP_ERR_BAD_SHAPE, "batch=%d outside [1, %d]", batch, kLayerMaxBatch);
  if (x == nullptr || K_cache == nullptr || V_cache == nullptr || pos == nullptr || ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "x, the caches, pos and ws must be non-NULL");
  if (!aligned16(x) || !aligned16(K_cache) || !aligned16(V_cache) || !aligned16(ws))
    return fail(POP_ERR_MISALIGNED, "x, the caches and ws must be 16-byte aligned");
  if (dense_ffn != 0 && dense_ffn != 1) return fail(POP_ERR_INVALID_ARGUMENT, "dense_ffn must be 0 or 1");
  const DecodeLayerWs lw = decode_layer_ws(batch, *s, dt, (char*)ws);
  if (ws_bytes < lw.total) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, lw.total);
  const size_t ffn_bytes = pop_decode_workspace_bytes(batch, s->d, s->d_ff);
  if (!dense_ffn) {  // the FFN step's own checks, before anything is enqueued
    if (!(r >= 0.0 && r < 1.0)) return fail(POP_ERR_INVALID_ARGUMENT, "r=%g outside [0, 1)", r);
    if (n_R < 0 || n_C < 0 || (int64_t)n_R + n_C > s->d_ff)
      return fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, n_C=%d inconsistent with d_ff=%d", n_R, n_C, s->d_ff);
    if ((n_R > 0 && R == nullptr) || (n_C > 0 && C == nullptr))
      return fail(POP_ERR_INVALID_ARGUMENT, "R or C is NULL with a nonzero size");
    if (kDebugLists) {
      const pop_status sd = debug_check_device_lists(R, n_R, C, n_C, s->d_ff, stream);
      if (sd != POP_OK) return sd;
    }
  }
  const DebugNested nest;  // R and C are checked above
  hipStream_t h = (hipStream_t)stream;
  trace_mark(h);
  if (dt == POP_BF16)
    enqueue_layer_decode_attention<bf16s>(h, x, batch, *s, w, K_cache, V_cache, pos, lw);
  else
    enqueue_layer_decode_attention<float>(h, x, batch, *s, w, K_cache, V_cache, pos, lw);
  const int D = s->d;
  const int64_t n = (int64_t)batch * D;
  // batch 1: the FFN's last kernel adds its output to x (= h) itself
  if (batch == 1 && decode_ffn_accumulate_b1(lw.xn, D, w->W_gate, w->W_up, w->W_downT, s->d_ff, dt, dense_ffn != 0, R,
                                             n_R, C, n_C, r, x, selected, lw.ffn, stream))
    return launched_layer();
  st = dense_ffn ? pop_dense_ffn_decode(lw.xn, batch, D, w->W_gate, w->W_up, w->W_downT, s->d_ff, dt, lw.y, lw.ffn,
                                        ffn_bytes, stream)
                 : pop_decode_ffn(lw.xn, batch, D, w->W_gate, w->W_up, w->W_downT, s->d_ff, dt, R, n_R, C, n_C, r,
                                  lw.y, selected, lw.ffn, ffn_bytes, stream);
  if (st != POP_OK) return st;
  POP_LAUNCH(k_add, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, h, x, (const float*)lw.y, n);
  return launched_layer();
}

extern "C" pop_status pop_layer_prefill(float* x, int32_t batch, int32_t n_tokens, const pop_layer_shape* s,
                                        const pop_layer_weights* w, pop_dtype dt, void* K_cache, void* V_cache,
                                        double r, double gamma, int32_t* R, int32_t* C, int32_t* P, float* importance,
                                        void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status st = check_layer(s, dt);
  if (st != POP_OK) return st;
  if ((st = check_weights(w)) != POP_OK) return st;
  if ((st = check_rate(r, gamma)) != POP_OK) return st;
  if (batch < 1 || n_tokens < 1 || n_tokens > s->cache_len || (int64_t)batch * n_tokens > (1 << 22))
    return fail(POP_ERR_BAD_SHAPE, "batch=%d, n_tokens=%d: need >= 1, n_tokens <= cache_len=%d, batch*n_tokens <= 2^22",
                batch, n_tokens, s->cache_len);
  if (x == nullptr || K_cache == nullptr || V_cache == nullptr || ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "x, the caches and ws must be non-NULL");
  if (!aligned16(x) || !aligned16(K_cache) || !aligned16(V_cache) || !aligned16(ws) || !aligned16(importance))
    return fail(POP_ERR_MISALIGNED, "x, the caches, importance and ws must be 16-byte aligned");
  const pop_counts c = counts(s->d_ff, r, gamma);
  if ((c.n_R > 0 && R == nullptr) || (c.n_C > 0 && C == nullptr) || (c.n_P > 0 && P == nullptr))
    return fail(POP_ERR_INVALID_ARGUMENT, "an output list with a nonzero size is NULL");
  const int64_t M = (int64_t)batch * n_tokens;
  const PrefillLayerWs lw = prefill_layer_ws(M, *s, dt, (char*)ws);
  if (ws_bytes < lw.total) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, lw.total);
  hipStream_t h = (hipStream_t)stream;
  const int D = s->d, Hd = s->n_heads * s->head_dim;
  trace_mark(h);
  if (dt == POP_BF16)
    POP_LAUNCH(k_rmsnorm<bf16s>, dim3((unsigned)M), dim3(256), 0, h, x, D, w->attn_norm, (float)s->eps, (bf16s*)lw.xn);
  else
    POP_LAUNCH(k_rmsnorm<float>, dim3((unsigned)M), dim3(256), 0, h, x, D, w->attn_norm, (float)s->eps, (float*)lw.xn);
  launch_gemm_kmajor(h, lw.xn, (int)M, D, w->Wqkv_T, D, n_qkv(*s), dt, lw.Y);
  const dim3 gq = qkv_grid(M, *s, 1);
  if (dt == POP_BF16) {
    POP_LAUNCH((k_qkv_rope<bf16s, 1>), gq, dim3(256), 0, h, lw.Y, 1, (int)M, s->n_heads, s->n_kv_heads, s->head_dim,
               n_tokens, 0, (const int32_t*)nullptr, s->rope_theta, s->cache_len, lw.q, (bf16s*)K_cache,
               (bf16s*)V_cache);
    launch_attn_prefill<bf16s>(h, *s, batch, n_tokens, K_cache, V_cache, lw);
  } else {
    POP_LAUNCH((k_qkv_rope<float, 1>), gq, dim3(256), 0, h, lw.Y, 1, (int)M, s->n_heads, s->n_kv_heads, s->head_dim,
               n_tokens, 0, (const int32_t*)nullptr, s->rope_theta, s->cache_len, lw.q, (float*)K_cache,
               (float*)V_cache);
    launch_attn_prefill<float>(h, *s, batch, n_tokens, K_cache, V_cache, lw);
  }
  launch_gemm_kmajor(h, lw.ao, (int)M, Hd, w->Wo_T, Hd, D, dt, lw.Y);
  const int64_t n = M * D;
  POP_LAUNCH(k_add, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, h, x, (const float*)lw.Y, n);
  if (dt == POP_BF16)
    POP_LAUNCH(k_rmsnorm<bf16s>, dim3((unsigned)M), dim3(256), 0, h, x, D, w->ffn_norm, (float)s->eps, (bf16s*)lw.xn);
  else
    POP_LAUNCH(k_rmsnorm<float>, dim3((unsigned)M), dim3(256), 0, h, x, D, w->ffn_norm, (float)s->eps, (float*)lw.xn);
  st = pop_prefill_ffn_partition(lw.xn, M, D, w->W_gate, w->W_up, w->W_downT, s->d_ff, dt, r, gamma, lw.Y, R, C, P,
                                 importance, lw.ffn, pop_prefill_ffn_partition_workspace_bytes(M, D, s->d_ff, dt),
                                 stream);
  if (st != POP_OK) return st;
  POP_LAUNCH(k_add, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, h, x, (const float*)lw.Y, n);
  return launched_layer();
}
