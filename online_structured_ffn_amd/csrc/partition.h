// Three-region split of n <= kPartMaxN channels by one workgroup (POP notes,
// "Key design 1": P = the c_low least important channels, C = the next
// c_high - c_low, R = the rest; each list in ascending channel order).
//
// Order: channel i has the value u_i = value_bits(I_i).  Ascending (least
// important first): smaller value first, on equal values the larger index
// first.  A cut at rank c puts the c least important channels below it.
//
// Layout: the keys sit in LDS, keys[i] for channel i.  Wave w of the
// workgroup visits channels [w * jw * 64, (w + 1) * jw * 64), lane l the
// channel w * jw * 64 + j * 64 + l at step j < jw, jw = ceil(n / NTH):
// consecutive lanes visit consecutive channels, so the stores of the lists are
// coalesced, and every ordered count across channels is a ballot within a step
// plus a scan over steps and waves.  One workgroup alone on a CU is bound by
// latency here: the passes over the keys are few (range, histogram, one gather
// for both cuts, classes, stores), each issues four independent LDS reads per
// lane at a time, and the loops stay rolled so that the code stays small.
//
// Finding the channel at a cut rank: histograms of 4096 bins over the value
// bits.  The first covers [min, max] of all keys (the bin of a key is
// (u - lo) >> shift with the least shift that fits 4096 bins), which places
// both cuts; each cut's bin is then refined the same way while it holds more
// than kPartResolve keys and more than one value (at most two more rounds for
// 31-bit values).  The keys of a bin of at most kPartResolve keys are ranked
// against each other directly.  Every loop is bounded, every LDS index lies in
// its array, and the result does not depend on timing: identical inputs give
// identical lists.
#pragma once

#include "pop_device.h"

namespace pop {

constexpr int kPartMaxN = 32768;
constexpr int kPartBins = 4096;
constexpr int kPartResolve = 256;  // a bin of at most this many keys is resolved directly
constexpr int kPartUnroll = 4;     // steps per pass iteration (independent LDS reads in flight)

template <int NTH>
struct PartShared {
  static constexpr int kWaves = NTH / 64;
  // keys of a bin resolved directly: one thread per key of each cut
  static constexpr int kRes = NTH / 2 < kPartResolve ? NTH / 2 : kPartResolve;
  unsigned int hist[kSelSlots];
  __align__(16) uint32_t rv[2][kRes];  // the keys of each cut's small bin (values, channels)
  __align__(16) int ri[2][kRes];
  int rcnt[2];
  uint32_t red[kWaves][2];
  int scan[kWaves][4];
  uint32_t tb[2][4];   // a cut's bin: lo, hi, rank inside the bin, keys in the bin
  uint32_t res[2][3];  // a resolved cut: value, q, m
};

// LDS bytes of a split of n channels by NTH threads: the keys (channel order,
// room for the unrolled passes' reads past the last step), then PartShared.
template <int NTH>
__host__ __device__ constexpr size_t part_keys_bytes(int n) {
  return ((size_t)((n + NTH - 1) / NTH) * NTH + 64 * kPartUnroll) * sizeof(uint32_t);
}
template <int NTH>
__host__ __device__ constexpr size_t part_lds_bytes(int n) {
  return part_keys_bytes<NTH>(n) + sizeof(PartShared<NTH>);
}

// The state of one cut while it is being found.
struct PartCut {
  uint32_t lo, hi;  // the values the cut's bin spans
  int rk;           // rank of the cut inside the bin
  int cnt;          // keys in the bin
  int beyond;       // the cut is at n: every key lies below it
  uint32_t v;       // resolved: the value at the cut,
  int q, m;         // the keys of value v below the cut, the keys of value v
};

// Sum over the waves' entries sh.scan[.][slot]: the part before this wave and
// the total.
template <int NTH>
__device__ __forceinline__ int part_wave_prefix(const PartShared<NTH>& sh, int slot, int wave, int& total) {
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const int x = sh.scan[w][slot];
    off += w < wave ? x : 0;
    tot += x;
  }
  total = tot;
  return off;
}

// One pass over this thread's steps j < jw, kPartUnroll at a time:
// f(j, idx, ok, u) with ok = (j < jw and idx < n).  Reads past the last step
// stay inside the keys' padding and are not used.
template <int NTH, typename F>
__device__ __forceinline__ void part_pass(const uint32_t* __restrict__ keys, int n, int jw, int base, F&& f) {
#pragma unroll 1
  for (int j0 = 0; j0 < jw; j0 += kPartUnroll) {
    uint32_t u[kPartUnroll];
#pragma unroll
    for (int t = 0; t < kPartUnroll; ++t) u[t] = keys[base + (j0 + t) * 64];
#pragma unroll
    for (int t = 0; t < kPartUnroll; ++t) {
      const int j = j0 + t, idx = base + j * 64;
      f(j, idx, j < jw && idx < n, u[t]);
    }
  }
}

// One histogram round over the keys in [L, H] for nr (1 or 2) ranks rA, rB
// inside [L, H]: on return sh.tb[t] (t < nr) describes the bin that holds
// rank t.  The histogram is zero on entry and on return.
template <int NTH>
__device__ __forceinline__ void part_round(const uint32_t* __restrict__ keys, int n, int jw, int base, uint32_t L,
                                           uint32_t H, int rA, int rB, int nr, PartShared<NTH>& sh) {
  constexpr int BPT = kPartBins / NTH;
  static_assert(kPartBins % NTH == 0 && BPT <= 16, "bins per thread");
  const int tid = threadIdx.x;
  const uint32_t span = H - L;
  const int bits = span ? 32 - __clz((int)span) : 0;  // span < 2^31
  const int shift = bits > 12 ? bits - 12 : 0;
  part_pass<NTH>(keys, n, jw, base, [&](int, int, bool ok, uint32_t u) {
    if (ok && u >= L && u <= H) atomicAdd(&sh.hist[sel_slot((int)((u - L) >> shift))], 1u);
  });
  __syncthreads();
  unsigned int hb[BPT];
  int local = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    hb[b] = sh.hist[sel_slot(tid * BPT + b)];
    local += (int)hb[b];
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int incl = wave_incl_scan(local);
  if (lane == 63) sh.scan[wave][0] = incl;
  __syncthreads();
  int total;
  const int excl = part_wave_prefix(sh, 0, wave, total) + incl - local;
  for (int t = 0; t < nr; ++t) {
    const int r = t ? rB : rA;
    if (r >= excl && r < excl + local) {
      int cum = excl;
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int c = (int)hb[b];
        if (r >= cum && r < cum + c) {
          const uint32_t blo = L + ((uint32_t)(tid * BPT + b) << shift);
          sh.tb[t][0] = blo;
          sh.tb[t][1] = min(H, blo + ((1u << shift) - 1u));
          sh.tb[t][2] = (uint32_t)(r - cum);
          sh.tb[t][3] = (uint32_t)c;
        }
        cum += c;
      }
    }
  }
  // this thread's bins back to zero (every read of them is above)
#pragma unroll
  for (int b = 0; b < BPT; ++b) sh.hist[sel_slot(tid * BPT + b)] = 0u;
  __syncthreads();
}

__device__ __forceinline__ void part_take_bin(PartCut& c, const uint32_t (&tb)[4]) {
  c.lo = tb[0];
  c.hi = tb[1];
  c.rk = (int)tb[2];
  c.cnt = (int)tb[3];
}

// Resolves the cuts whose bins hold more than one value (at most
// PartShared::kRes keys each): one gather of both bins' keys, then every
// gathered key ranks itself against the others of its bin (cut 0 on threads
// [0, kRes), cut 1 on [NTH / 2, NTH / 2 + kRes)).  A cut whose bin holds one
// value is complete without it.  sh.rcnt must be zero on entry.
template <int NTH>
__device__ __forceinline__ void part_resolve(const uint32_t* __restrict__ keys, int n, int jw, int base, PartCut& c0,
                                             PartCut& c1, PartShared<NTH>& sh) {
  constexpr int kRes = PartShared<NTH>::kRes;
  const int tid = threadIdx.x;
  const bool g0 = !c0.beyond && c0.lo != c0.hi;
  const bool g1 = !c1.beyond && c1.lo != c1.hi;
  if (!c0.beyond && !g0) {
    c0.v = c0.lo;
    c0.q = c0.rk;
    c0.m = c0.cnt;
  }
  if (!c1.beyond && !g1) {
    c1.v = c1.lo;
    c1.q = c1.rk;
    c1.m = c1.cnt;
  }
  if (!g0 && !g1) return;  // block-uniform
  part_pass<NTH>(keys, n, jw, base, [&](int, int idx, bool ok, uint32_t u) {
    if (ok && g0 && u >= c0.lo && u <= c0.hi) {
      const int slot = atomicAdd(&sh.rcnt[0], 1);
      if (slot < kRes) {
        sh.rv[0][slot] = u;
        sh.ri[0][slot] = idx;
      }
    }
    if (ok && g1 && u >= c1.lo && u <= c1.hi) {
      const int slot = atomicAdd(&sh.rcnt[1], 1);
      if (slot < kRes) {
        sh.rv[1][slot] = u;
        sh.ri[1][slot] = idx;
      }
    }
  });
  __syncthreads();
  // neutral padding up to a multiple of 4 (a value above every key counts in
  // none of the sums below)
  const int m0 = g0 ? min(c0.cnt, kRes) : 0, m1 = g1 ? min(c1.cnt, kRes) : 0;
  const int p0 = (m0 + 3) & ~3, p1 = (m1 + 3) & ~3;
  if (tid < p0 - m0) {
    sh.rv[0][m0 + tid] = 0xffffffffu;
    sh.ri[0][m0 + tid] = -1;
  }
  if (tid >= 64 && tid - 64 < p1 - m1) {
    sh.rv[1][m1 + tid - 64] = 0xffffffffu;
    sh.ri[1][m1 + tid - 64] = -1;
  }
  __syncthreads();
  const int side = tid >= NTH / 2 ? 1 : 0;
  const int k = tid - side * (NTH / 2);
  const int mb = side ? m1 : m0, pb = side ? p1 : p0;
  if (k < mb) {
    const int crk = side ? c1.rk : c0.rk;
    const uint32_t vv = sh.rv[side][k];
    const int ii = sh.ri[side][k];
    int below = 0, lt = 0, eqn = 0;
#pragma unroll 1
    for (int e = 0; e < pb; e += 4) {
      const uint4 ve = *reinterpret_cast<const uint4*>(&sh.rv[side][e]);
      const int4 ie = *reinterpret_cast<const int4*>(&sh.ri[side][e]);
      lt += (ve.x < vv) + (ve.y < vv) + (ve.z < vv) + (ve.w < vv);
      eqn += (ve.x == vv) + (ve.y == vv) + (ve.z == vv) + (ve.w == vv);
      below += (ve.x < vv || (ve.x == vv && ie.x > ii)) + (ve.y < vv || (ve.y == vv && ie.y > ii)) +
               (ve.z < vv || (ve.z == vv && ie.z > ii)) + (ve.w < vv || (ve.w == vv && ie.w > ii));
    }
    if (below == crk) {
      sh.res[side][0] = vv;
      sh.res[side][1] = (uint32_t)(crk - lt);
      sh.res[side][2] = (uint32_t)eqn;
    }
  }
  __syncthreads();
  if (g0) {
    c0.v = sh.res[0][0];
    c0.q = (int)sh.res[0][1];
    c0.m = (int)sh.res[0][2];
  }
  if (g1) {
    c1.v = sh.res[1][0];
    c1.q = (int)sh.res[1][1];
    c1.m = (int)sh.res[1][2];
  }
}

// Whether a key of value u with eq_after equal keys at larger indices lies
// below the resolved cut c.
__device__ __forceinline__ bool part_below(const PartCut& c, uint32_t u, int eq_after) {
  return c.beyond || u < c.v || (u == c.v && eq_after < c.q);
}

// The split itself.  keys: LDS of part_keys_bytes<NTH>(n) bytes, keys[i] =
// value_bits(I_i) for i < n (the rest is never used); 1 <= n <= kPartMaxN.
// mn, mx: the least and largest of the keys this thread stored (any split of
// the keys over the threads; 0xffffffff and 0 for none).  Lists: R
// (n - c_high), C (c_high - c_low), P (c_low) entries.  The first barrier
// below orders the caller's stores of keys.  Ends with a barrier-free store
// phase: keys and sh may be reused only after a barrier.
template <int NTH, typename Emit>
__device__ __forceinline__ void split_block(const uint32_t* __restrict__ keys, int n, uint32_t mn, uint32_t mx,
                                            int c_low, int c_high, Emit&& emit, PartShared<NTH>& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int jw = (n + NTH - 1) / NTH;
  const int base = wave * jw * 64 + lane;
  const uint64_t lanes_below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const uint64_t lanes_above = lane < 63 ? (~0ull << (lane + 1)) : 0ull;
  // ordered by the barrier below
  for (int i = tid; i < kSelSlots; i += NTH) sh.hist[i] = 0u;
  if (tid < 2) sh.rcnt[tid] = 0;
  // ---- range of the values
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  if (lane == 0) {
    sh.red[wave][0] = mn;
    sh.red[wave][1] = mx;
  }
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    mn = min(mn, sh.red[w][0]);
    mx = max(mx, sh.red[w][1]);
  }
  // ---- the two cuts: one histogram round over [mn, mx] places both
  PartCut c0{mn, mx, c_low, n, c_low >= n ? 1 : 0, 0u, 0, 0};
  PartCut c1{mn, mx, c_high, n, c_high >= n ? 1 : 0, 0u, 0, 0};
  if (!c0.beyond || !c1.beyond) {  // block-uniform
    const int nr = (!c0.beyond && !c1.beyond) ? 2 : 1;
    part_round<NTH>(keys, n, jw, base, mn, mx, c0.beyond ? c1.rk : c0.rk, c1.rk, nr, sh);
    if (!c0.beyond) part_take_bin(c0, sh.tb[0]);
    if (!c1.beyond) part_take_bin(c1, sh.tb[nr - 1]);
  }
  // a bin of more than kRes keys and more than one value is narrowed by
  // further rounds: at most two per cut (a first-round bin spans at most
  // 2^19 values, a second-round bin at most 2^7, a third-round bin one value)
  constexpr int kRes = PartShared<NTH>::kRes;
#pragma unroll 1
  for (int it = 0; it < 4; ++it) {  // block-uniform
    const bool n0 = !c0.beyond && c0.lo != c0.hi && c0.cnt > kRes;
    const bool n1 = !c1.beyond && c1.lo != c1.hi && c1.cnt > kRes;
    if (!n0 && !n1) break;
    part_round<NTH>(keys, n, jw, base, n0 ? c0.lo : c1.lo, n0 ? c0.hi : c1.hi, n0 ? c0.rk : c1.rk, 0, 1, sh);
    if (n0)
      part_take_bin(c0, sh.tb[0]);
    else
      part_take_bin(c1, sh.tb[0]);
  }
  part_resolve<NTH>(keys, n, jw, base, c0, c1, sh);
  // ---- equal keys at larger indices, for a cut inside a run of equal values
  const bool split0 = !c0.beyond && c0.q > 0 && c0.q < c0.m;
  const bool split1 = !c1.beyond && c1.q > 0 && c1.q < c1.m;
  int after0 = 0, after1 = 0;
  if (split0 || split1) {  // block-uniform
    int e0 = 0, e1 = 0;
    part_pass<NTH>(keys, n, jw, base, [&](int, int, bool ok, uint32_t u) {
      e0 += __popcll(__ballot(ok && u == c0.v));
      e1 += __popcll(__ballot(ok && u == c1.v));
    });
    if (lane == 0) {
      sh.scan[wave][0] = e0;
      sh.scan[wave][1] = e1;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
      after0 += w > wave ? sh.scan[w][0] : 0;
      after1 += w > wave ? sh.scan[w][1] : 0;
    }
    __syncthreads();
  }
  // ---- classes (0 = P, 1 = C, 2 = R)
  uint64_t cls = 0;  // 2 bits per step
  int cc0 = 0, cc1 = 0, cc2 = 0;
  if (!split0 && !split1) {  // block-uniform
    // no run of equal values straddles a cut: below cut t is u < t0 (u <= v
    // when every key of value v lies below, q == m)
    const uint32_t t0 = c0.beyond ? 0xffffffffu : c0.v + (c0.q == c0.m ? 1u : 0u);
    const uint32_t t1 = c1.beyond ? 0xffffffffu : c1.v + (c1.q == c1.m ? 1u : 0u);
    part_pass<NTH>(keys, n, jw, base, [&](int j, int, bool ok, uint32_t u) {
      const uint32_t c = u < t0 ? 0u : (u < t1 ? 1u : 2u);
      cls |= (uint64_t)c << (2 * j);
      const uint64_t all = __ballot(ok);
      const uint64_t k0 = __ballot(ok && c == 0u), k1 = __ballot(ok && c == 1u);
      cc0 += __popcll(k0);
      cc1 += __popcll(k1);
      cc2 += __popcll(all & ~(k0 | k1));
    });
  } else {
    // from the last step down, so that the equal keys at larger indices are
    // counted as they are passed
    const int jtop = (jw + kPartUnroll - 1) / kPartUnroll * kPartUnroll;
#pragma unroll 1
    for (int j0 = jtop - kPartUnroll; j0 >= 0; j0 -= kPartUnroll) {
      uint32_t uu[kPartUnroll];
#pragma unroll
      for (int t = 0; t < kPartUnroll; ++t) uu[t] = keys[base + (j0 + t) * 64];
#pragma unroll
      for (int t = kPartUnroll - 1; t >= 0; --t) {
        const int j = j0 + t, idx = base + j * 64;
        const bool ok = j < jw && idx < n;
        const uint32_t u = uu[t];
        const uint64_t q0 = __ballot(ok && u == c0.v);
        const uint64_t q1 = __ballot(ok && u == c1.v);
        const bool b0 = part_below(c0, u, after0 + __popcll(q0 & lanes_above));
        const bool b1 = part_below(c1, u, after1 + __popcll(q1 & lanes_above));
        after0 += __popcll(q0);
        after1 += __popcll(q1);
        const uint32_t c = b0 ? 0u : (b1 ? 1u : 2u);
        cls |= (uint64_t)c << (2 * j);
        const uint64_t all = __ballot(ok);
        const uint64_t k0 = __ballot(ok && c == 0u), k1 = __ballot(ok && c == 1u);
        cc0 += __popcll(k0);
        cc1 += __popcll(k1);
        cc2 += __popcll(all & ~(k0 | k1));
      }
    }
  }
  if (lane == 0) {
    sh.scan[wave][0] = cc0;
    sh.scan[wave][1] = cc1;
    sh.scan[wave][2] = cc2;
  }
  __syncthreads();
  int tot;
  int run0 = part_wave_prefix(sh, 0, wave, tot);
  int run1 = part_wave_prefix(sh, 1, wave, tot);
  int run2 = part_wave_prefix(sh, 2, wave, tot);
  // ---- ordered, coalesced stores: emit(class, position in its list, channel)
  for (int j = 0; j < jw; ++j) {
    const int idx = base + j * 64;
    const bool ok = idx < n;
    const uint32_t c = (uint32_t)(cls >> (2 * j)) & 3u;
    const uint64_t all = __ballot(ok);
    const uint64_t k0 = __ballot(ok && c == 0u), k1 = __ballot(ok && c == 1u);
    const uint64_t k2 = all & ~(k0 | k1);
    const uint64_t mine = c == 0u ? k0 : (c == 1u ? k1 : k2);
    const int run = c == 0u ? run0 : (c == 1u ? run1 : run2);
    if (ok) emit(c, run + __popcll(mine & lanes_below), idx);
    run0 += __popcll(k0);
    run1 += __popcll(k1);
    run2 += __popcll(k2);
  }
}

// The three-region split: P the c_low least important, C the next
// c_high - c_low, R the rest, each ascending (positions capped at the list
// sizes; an exact split never reaches the caps).  Arguments as split_block.
template <int NTH>
__device__ __forceinline__ void partition_block(const uint32_t* __restrict__ keys, int n, uint32_t mn, uint32_t mx,
                                                int c_low, int c_high, int32_t* __restrict__ R,
                                                int32_t* __restrict__ C, int32_t* __restrict__ P,
                                                PartShared<NTH>& sh) {
  const int n_P = c_low, n_C = c_high - c_low, n_R = n - c_high;
  split_block<NTH>(keys, n, mn, mx, c_low, c_high, [=](uint32_t c, int pos, int idx) {
    if (c == 0u) {
      if (pos < n_P) P[pos] = idx;
    } else if (c == 1u) {
      if (pos < n_C) C[pos] = idx;
    } else {
      if (pos < n_R) R[pos] = idx;
    }
  }, sh);
}

// LDS bytes of topk_select<NTH> over n scores.
template <int NTH>
__host__ __device__ constexpr size_t topk_lds_bytes(int n) {
  return part_lds_bytes<NTH>(n);
}

// S = the k most important of n candidates (score descending, position
// ascending on ties: the order of the split), written in ascending order as
// positions into C and, when `selected` is not NULL, as channels C[position].
// One workgroup; 1 <= n <= kPartMaxN; smem: topk_lds_bytes<NTH>(n) bytes,
// 16-byte aligned.  Scores are |z| >= 0.
template <int NTH>
__device__ __forceinline__ void topk_select(const float* __restrict__ score, int n, int k,
                                            const int32_t* __restrict__ C, int32_t* __restrict__ positions,
                                            int32_t* __restrict__ selected, unsigned char* smem) {
  if (n <= 0 || k <= 0) return;
  k = min(k, n);
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
  PartShared<NTH>& sh = *reinterpret_cast<PartShared<NTH>*>(smem + part_keys_bytes<NTH>(n));
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll 4
  for (int i = threadIdx.x; i < n; i += NTH) {
    const uint32_t u = value_bits(score[i]);
    keys[i] = u;
    mn = min(mn, u);
    mx = max(mx, u);
  }
  // the k most important: the channels at or above the cut of rank n - k
  split_block<NTH>(keys, n, mn, mx, n - k, n, [=](uint32_t c, int pos, int idx) {
    if (c == 1u && pos < k) {
      positions[pos] = idx;
      if (selected != nullptr) selected[pos] = C[idx];
    }
  }, sh);
}

}  // namespace pop
