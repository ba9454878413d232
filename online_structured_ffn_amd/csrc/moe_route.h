// Top-2 routing for the mixture-of-experts form of the path (the POP notes
// evaluate MoE models; every expert keeps its own partition).  Reading taken:
// a token goes to the experts of its two largest router logits (ties to the
// lower expert id), weighted by the softmax of those two logits.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pop_device.h"

namespace pop {

constexpr int kMoeMaxExperts = 64;
constexpr int kBucketThreads = 256;

// One thread per token.  ex[2t] is the best expert, ex[2t + 1] the second;
// wt (may be NULL) their weights.
template <int kUnused = 0>
__global__ __launch_bounds__(256) void k_moe_top2(const float* __restrict__ logits, int T, int E,
                                                  int32_t* __restrict__ ex, float* __restrict__ wt) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* l = logits + (int64_t)t * E;
  float b1 = l[0], b2 = -INFINITY;
  int e1 = 0, e2 = 1;
  for (int e = 1; e < E; ++e) {
    const float v = l[e];
    if (v > b1) {
      b2 = b1;
      e2 = e1;
      b1 = v;
      e1 = e;
    } else if (v > b2) {
      b2 = v;
      e2 = e;
    }
  }
  ex[2 * t] = e1;
  ex[2 * t + 1] = e2;
  if (wt != nullptr) {
    const float g = expf(b2 - b1);  // in (0, 1]
    wt[2 * t] = 1.0f / (1.0f + g);
    wt[2 * t + 1] = g / (1.0f + g);
  }
}

// Groups the 2T (token, expert) pairs by expert, tokens ascending within each
// expert.  One workgroup: thread j owns tokens [j * per, (j + 1) * per) and
// counts its pairs per expert in cnt[e][j]; an exclusive scan over cnt in
// (expert, thread) order gives each (expert, thread) its first position.
//   offsets[e] .. offsets[e + 1]: the pairs of expert e in tokens[];
//   slot[2t + j]: where the pair (t, ex[2t + j]) sits in tokens[].
template <int kUnused = 0>
__global__ __launch_bounds__(kBucketThreads) void k_moe_bucket(const int32_t* __restrict__ ex, int T, int E,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ tokens,
                                                               int32_t* __restrict__ slot) {
  constexpr int NTH = kBucketThreads;
  __shared__ int cnt[kMoeMaxExperts * NTH];
  __shared__ int wtot[NTH / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (T + NTH - 1) / NTH;
  const int t0 = min(T, tid * per), t1 = min(T, t0 + per);
  for (int e = 0; e < E; ++e) cnt[e * NTH + tid] = 0;
  for (int t = t0; t < t1; ++t) {
    ++cnt[ex[2 * t] * NTH + tid];
    ++cnt[ex[2 * t + 1] * NTH + tid];
  }
  __syncthreads();
  // exclusive scan of the flattened cnt: thread j sums entries [j * E, (j + 1) * E)
  int s = 0;
  for (int i = 0; i < E; ++i) s += cnt[tid * E + i];
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int run = incl - s;
  for (int w = 0; w < wave; ++w) run += wtot[w];
  for (int i = 0; i < E; ++i) {
    const int c = cnt[tid * E + i];
    cnt[tid * E + i] = run;
    run += c;
  }
  __syncthreads();
  if (tid < E) offsets[tid] = cnt[tid * NTH];
  if (tid == 0) offsets[E] = 2 * T;
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = ex[2 * t + j];
      const int p = cnt[e * NTH + tid]++;
      tokens[p] = t;
      slot[2 * t + j] = p;
    }
  }
}

}  // namespace pop
