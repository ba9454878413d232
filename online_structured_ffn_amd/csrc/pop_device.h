// Device-side helpers shared by the libpop kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pop {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage type for bf16 elements; arithmetic is always done in fp32.
struct bf16s {
  uint16_t bits;
};

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;  // elements per 16-byte load
};
template <>
struct Vec<bf16s> {
  static constexpr int N = 8;
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streamed once per call: keep it out of the caches' reuse set.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---- data handed between workgroups of one launch
// Agent-scope relaxed atomics: every access below goes to the device's
// coherence point, so a value one workgroup stores is the value another
// workgroup loads, whichever XCD (and L2) each runs on.  No release or acquire
// fence is used (a device-scope release writes back the whole L2 of the XCD and
// costs microseconds per workgroup); a reader learns that data is there from a
// valid bit carried in the same 64-bit word as the data it guards, so no
// order between stores to different locations is assumed.
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_coh(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// accesses (lgkmcnt(0); vmcnt and expcnt left at their maxima in the gfx9
// encoding), then meets the others.  Unlike __syncthreads() it does not wait
// for the wave's global loads in flight, so loads issued before it stay in
// flight across it.  Global memory written before it is not made visible to
// the other waves by it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Polls *p (coherent) until pred(value) holds, at most `limit` times, sleeping
// briefly between polls; returns the last value read and sets ok.
template <typename T, typename Pred>
__device__ __forceinline__ T poll_coh(const T* p, Pred pred, int limit, bool& ok) {
  T v = ld_coh(p);
  int n = 0;
  while (!pred(v) && ++n < limit) {
    __builtin_amdgcn_s_sleep(2);
    v = ld_coh(p);
  }
  ok = pred(v);
  return v;
}

__device__ __forceinline__ void unpack(const u32x4 v, float (&f)[8], bf16s) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(v[j] << 16);
    f[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(const u32x4 v, float (&f)[4], float) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(v[j]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Wave64 sum through DPP row/bank operations (no LDS round trips).  The
// total is exact in lane 63; other lanes hold partial sums.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum_last(float v) {
  v += dpp_mov<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141, 0xf>(v);  // row_half_mirror: 8-lane sums
  v += dpp_mov<0x140, 0xf>(v);  // row_mirror: 16-lane sums
  v += dpp_mov<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_mov<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;                     // lane 63: sum of all 64 lanes
}
// The wave total broadcast to every lane.
__device__ __forceinline__ float wave_sum_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum_last(v)), 63));
}

__device__ __forceinline__ float silu(float a) {
  // a * sigmoid(a); expf(-a) overflows to +inf for a < -88 and the quotient is -0.
  return a / (1.0f + expf(-a));
}

// Ordered bits of a non-negative float (-0 folded onto +0): larger value,
// larger unsigned integer.
__device__ __forceinline__ uint32_t value_bits(float v) { return __float_as_uint(v) & 0x7fffffffu; }

// ---------------------------------------------------------------------------
// One-workgroup exact selection over n <= MAXN keys.
//
// Element i (0 <= i < n) has the 64-bit key (value_bits << 32) | (0xffffffff - i):
// a larger value is more important and, on equal values, the lower index is.
// All keys are distinct.  For each of NT <= 2 targets (ascending ranks c) the
// select finds the value v of the key of rank c, the number m of elements
// whose value is v, and q, how many of those lie below rank c (they are the q
// equal elements with the largest indices).  "Below target t" then reads
//   value < v,  or  value == v and fewer than q equal elements have a larger index,
// which holds for exactly c elements.
//
// Thread t holds the values of its elements [t*E, min(n, (t+1)*E)),
// E = ceil(n / NTH), in registers.  The value bits are resolved from the top,
// below the leading bits that all n values share (one OR/AND reduction), in at
// most three radix passes of 12, 11 and up to 8 bits: each pass counts digits
// into an LDS histogram with atomics, and one block scan over the bins (DPP
// within a wave, LDS across waves) finds each target's bin.  Every loop is
// bounded and every LDS index lies inside its array.
// ---------------------------------------------------------------------------
constexpr int kSelMaxN = 32768;
constexpr int kSelBins = 4096;
// LDS slot of histogram bin g: one pad word per 32 bins, so that the threads
// of a wave reading their own runs of consecutive bins hit distinct banks.
__host__ __device__ constexpr int sel_slot(int g) { return g + (g >> 5); }
constexpr int kSelSlots = kSelBins + kSelBins / 32;

struct SelTarget {
  uint32_t prefix;  // value bits resolved so far (the whole value v once shift == 0)
  int shift;        // value bits below shift are still open
  int rank;         // rank still to find inside the current bucket (q once shift == 0)
  int count;        // elements in the current bucket (m once shift == 0)
  int beyond;       // rank >= n: every element is below
};

// A bucket of at most kSelResolve keys is resolved directly (every key of the
// bucket ranks itself against the others) instead of by further radix passes.
constexpr int kSelResolve = 64;

template <int NTH, int MAXN = kSelMaxN>
struct SelShared {
  static constexpr int kPerThread = (MAXN + NTH - 1) / NTH;
  unsigned int hA[kSelSlots];
  unsigned int hB[kSelSlots];
  SelTarget tgt[2];
  uint32_t red[NTH / 64][2];
  int scan[NTH / 64][3];
  uint32_t rv[kSelResolve];  // a small bucket's values and indices
  int ri[kSelResolve];
  int rcnt;
};

// DPP move within a wave; lanes whose source is outside the row, and rows
// outside ROW_MASK, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (no LDS).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111, 0xf>(v);  // row_shr:1
  v += dpp_i<0x112, 0xf>(v);  // row_shr:2
  v += dpp_i<0x114, 0xf>(v);  // row_shr:4
  v += dpp_i<0x118, 0xf>(v);  // row_shr:8   (prefix sums within each row of 16)
  v += dpp_i<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Bitwise OR over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= (uint32_t)dpp_i<0xb1, 0xf>((int)v);   // quad_perm [1,0,3,2]
  v |= (uint32_t)dpp_i<0x4e, 0xf>((int)v);   // quad_perm [2,3,0,1]
  v |= (uint32_t)dpp_i<0x141, 0xf>((int)v);  // row_half_mirror
  v |= (uint32_t)dpp_i<0x140, 0xf>((int)v);  // row_mirror: every lane holds its row's OR
  return (uint32_t)(__builtin_amdgcn_readlane((int)v, 0) | __builtin_amdgcn_readlane((int)v, 16) |
                    __builtin_amdgcn_readlane((int)v, 32) | __builtin_amdgcn_readlane((int)v, 48));
}

// Block-wide exclusive scan of one int per thread; returns the exclusive
// prefix and (through total) the block sum.  One barrier; sh.scan may be
// written again only after a later barrier.
template <int NTH, int MAXN>
__device__ __forceinline__ int block_excl_scan1(int v, int& total, SelShared<NTH, MAXN>& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) sh.scan[wave][0] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const int x = sh.scan[w][0];
    off += w < wave ? x : 0;
    tot += x;
  }
  total = tot;
  return off + incl - v;
}

// Block-wide exclusive scan of three per-thread counters (two barriers).
template <int NTH, int MAXN>
__device__ __forceinline__ void block_exclusive_scan3(int (&v)[3], int (&total)[3], SelShared<NTH, MAXN>& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) incl[j] = wave_incl_scan(v[j]);
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < 3; ++j) sh.scan[wave][j] = incl[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
      const int x = sh.scan[w][j];
      off += w < wave ? x : 0;
      tot += x;
    }
    v[j] = off + incl[j] - v[j];
    total[j] = tot;
  }
  __syncthreads();
}

// Loads value_bits(src[base + j]) for j < E into registers (n >= 1).
template <int EM>
__device__ __forceinline__ void sel_load_regs(const float* __restrict__ src, int n, int base, int E,
                                              uint32_t (&v)[EM]) {
#pragma unroll
  for (int j = 0; j < EM; ++j) v[j] = j < E ? value_bits(src[min(base + j, n - 1)]) : 0u;
}

// The select itself (see above).  v holds this thread's values; on return
// every thread's t[] holds the resolved targets (v, q, m in prefix, rank,
// count).  Ends with a barrier.
template <int NTH, int NT, int EM, int MAXN>
__device__ void select_targets(const uint32_t (&v)[EM], int n, int base, int E, const int (&ranks)[NT],
                               SelShared<NTH, MAXN>& sh, SelTarget (&t)[NT]) {
  static_assert(NT >= 1 && NT <= 2, "one or two targets");
  static_assert(kSelBins % NTH == 0 && kSelBins / NTH <= 16, "bins per thread");
  constexpr int BPT = kSelBins / NTH;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cnt = max(0, min(E, n - base));  // this thread's elements
  for (int i = tid; i < kSelSlots; i += NTH) {
    sh.hA[i] = 0u;
    sh.hB[i] = 0u;
  }
  // ---- leading bits shared by all values
  uint32_t o = 0u, a = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    if (j >= E) break;  // block-uniform
    o |= j < cnt ? v[j] : 0u;
    a &= j < cnt ? v[j] : 0xffffffffu;
  }
  o = wave_or(o);
  a = ~wave_or(~a);
  if (lane == 0) {
    sh.red[wave][0] = o;
    sh.red[wave][1] = a;
  }
  __syncthreads();  // also orders the histogram clears before the first pass
  uint32_t O = 0u, A = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    O |= sh.red[w][0];
    A &= sh.red[w][1];
  }
  const uint32_t diff = O ^ A;                      // values are 31-bit: diff < 2^31
  const int top = diff ? 32 - __clz((int)diff) : 0;  // bits >= top are common
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    t[i].prefix = top >= 31 ? 0u : (A >> top) << top;
    t[i].shift = top;
    t[i].rank = ranks[i];
    t[i].count = n;
    t[i].beyond = ranks[i] >= n ? 1 : 0;
  }
  // ---- radix passes
  const int widths[3] = {12, 11, 8};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    bool active = false;
#pragma unroll
    for (int i = 0; i < NT; ++i) active |= !t[i].beyond && t[i].shift > 0;
    if (!active) break;  // block-uniform
    const int shift = t[0].beyond ? t[NT - 1].shift : t[0].shift;  // the same for every active target
    const int wdt = min(widths[p], shift);
    const int s_new = shift - wdt;
    const uint32_t mask = (1u << wdt) - 1u;
    unsigned int* h = p == 1 ? sh.hB : sh.hA;
    const int per_t = p == 0 ? kSelBins : (p == 1 ? 2048 : 256);  // bins per target's section
    if (p == 1) {
      // pass 3 counts into hA again: clear it (pass 1's reads of hA ended at
      // the previous barrier; pass 3 starts two barriers later)
      for (int i = tid; i < kSelSlots; i += NTH) sh.hA[i] = 0u;
    }
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      if (j >= E) break;  // block-uniform
      if (j < cnt) {
        const uint32_t val = v[j];
        const int dg = (int)((val >> s_new) & mask);
        if (p == 0) {
          atomicAdd(&h[sel_slot(dg)], 1u);
        } else {
#pragma unroll
          for (int i = 0; i < NT; ++i)
            if (!t[i].beyond && t[i].shift > 0 && (val >> shift) == (t[i].prefix >> shift))
              atomicAdd(&h[sel_slot(i * per_t + dg)], 1u);
        }
      }
    }
    __syncthreads();
    // this thread's bins [tid * BPT, tid * BPT + BPT)
    unsigned int hb[BPT];
    int local = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      hb[b] = h[sel_slot(tid * BPT + b)];
      local += (int)hb[b];
    }
    int total;
    const int excl = block_excl_scan1(local, total, sh);
    const int sec0 = (p > 0 && !t[0].beyond) ? t[0].count : 0;  // elements counted in target 0's section
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (t[i].beyond || t[i].shift == 0) continue;
      const int r = t[i].rank + (i == 1 && p > 0 ? sec0 : 0);
      if (r >= excl && r < excl + local) {
        int cum = excl;
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          const int c = (int)hb[b];
          if (r >= cum && r < cum + c) {
            const int g = tid * BPT + b - (p > 0 ? i * per_t : 0);  // bin inside the target's section
            SelTarget u = t[i];
            u.prefix = t[i].prefix | ((uint32_t)g << s_new);
            u.shift = s_new;
            u.rank = r - cum;
            u.count = c;
            sh.tgt[i] = u;
          }
          cum += c;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (!t[i].beyond && t[i].shift > 0) t[i] = sh.tgt[i];
    // ---- small buckets: the key of rank t.rank inside the bucket, directly.
    // Ascending order (least important first): smaller value first, and on
    // equal values the larger index first.  The target's value v, its
    // multiplicity m (every key of value v lies in the bucket) and q = the
    // keys of value v below the target rank complete the target as the last
    // radix pass would.  Only when every open target's bucket is small: the
    // passes above move all open targets in step (one shift, one histogram
    // section per target).
    bool small = true;
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (!t[i].beyond && t[i].shift > 0) small &= t[i].count <= kSelResolve;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (!small || t[i].beyond || t[i].shift == 0) continue;  // block-uniform
      if (tid == 0) sh.rcnt = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EM; ++j) {
        if (j >= E) break;  // block-uniform
        if (j < cnt && (v[j] >> t[i].shift) == (t[i].prefix >> t[i].shift)) {
          const int slot = atomicAdd(&sh.rcnt, 1);
          if (slot < kSelResolve) {
            sh.rv[slot] = v[j];
            sh.ri[slot] = base + j;
          }
        }
      }
      __syncthreads();
      const int mb = t[i].count;  // == sh.rcnt
      if (tid < mb) {
        const uint32_t vv = sh.rv[tid];
        const int ii = sh.ri[tid];
        int below = 0, lt = 0, eqn = 0;
        for (int e = 0; e < mb; ++e) {
          const uint32_t ve = sh.rv[e];
          lt += ve < vv ? 1 : 0;
          eqn += ve == vv ? 1 : 0;
          below += (ve < vv || (ve == vv && sh.ri[e] > ii)) ? 1 : 0;
        }
        if (below == t[i].rank) {
          SelTarget u;
          u.prefix = vv;
          u.shift = 0;
          u.rank = t[i].rank - lt;
          u.count = eqn;
          u.beyond = 0;
          sh.tgt[i] = u;
        }
      }
      __syncthreads();
      t[i] = sh.tgt[i];
    }
  }
  __syncthreads();  // sh.tgt and the histograms may be reused after this
}

// Whether an element of value val with eq_after equal elements at larger
// indices lies below the resolved target t.
__device__ __forceinline__ bool sel_below(const SelTarget& t, uint32_t val, int eq_after) {
  if (t.beyond) return true;
  return val < t.prefix || (val == t.prefix && eq_after < t.rank);
}

// Counts of equal-valued elements before this thread's range, for targets
// whose equal group is split by the cut (0 < q < m); others get 0.  The scan
// runs only when some target needs it (block-uniform).
template <int NTH, int NT, int EM, int MAXN>
__device__ __forceinline__ void sel_eq_before(const uint32_t (&v)[EM], int E, int cnt, const SelTarget (&t)[NT],
                                              SelShared<NTH, MAXN>& sh, int (&eqb)[2]) {
  eqb[0] = eqb[1] = 0;
  bool need = false;
#pragma unroll
  for (int i = 0; i < NT; ++i) need |= !t[i].beyond && t[i].rank > 0 && t[i].rank < t[i].count;
  if (!need) return;
  int c[3] = {0, 0, 0};
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    if (j >= E) break;  // block-uniform
#pragma unroll
    for (int i = 0; i < NT; ++i) c[i] += (j < cnt && v[j] == t[i].prefix) ? 1 : 0;
  }
  int tot[3];
  block_exclusive_scan3(c, tot, sh);
  eqb[0] = c[0];
  eqb[1] = c[1];
}

// S = the k most important of n candidates (score descending, position
// ascending on ties), written in ascending order as positions into C and, when
// `selected` is not NULL, as channels C[position].  One workgroup; n <= MAXN.
template <int NTH, int MAXN>
__device__ __forceinline__ void topk_block(const float* __restrict__ score, int n, int k, const int32_t* __restrict__ C,
                           int32_t* __restrict__ positions, int32_t* __restrict__ selected, SelShared<NTH, MAXN>& sh) {
  constexpr int EM = SelShared<NTH, MAXN>::kPerThread;
  if (n <= 0 || k <= 0) return;
  k = min(k, n);
  const int E = (n + NTH - 1) / NTH;
  const int base = threadIdx.x * E;
  const int cnt = max(0, min(E, n - base));
  // This thread's channels come with its scores, so the final write waits on
  // no further global load.  When the keys fit the histogram buffers, scores
  // and channels are read coalesced (element tid + j * NTH) and handed to
  // their owners through LDS: a block sharing its CU with streaming work then
  // waits on few memory requests.
  int cv[EM];
  uint32_t v[EM];
  if constexpr (sel_slot(MAXN - 1) < kSelSlots) {
    uint32_t a[EM];
    int c[EM];
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      const int i = min((int)threadIdx.x + j * NTH, n - 1);
      a[j] = value_bits(score[i]);
      c[j] = selected != nullptr ? C[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      const int i = (int)threadIdx.x + j * NTH;
      if (i < n) {
        sh.hA[sel_slot(i)] = a[j];
        sh.hB[sel_slot(i)] = (unsigned int)c[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      const int i = min(base + j, n - 1);
      v[j] = sh.hA[sel_slot(i)];
      cv[j] = (int)sh.hB[sel_slot(i)];
    }
    __syncthreads();  // the select clears the buffers next
  } else {
    if (selected != nullptr) {
#pragma unroll
      for (int j = 0; j < EM; ++j) cv[j] = j < E ? C[min(base + j, n - 1)] : 0;
    }
    sel_load_regs(score, n, base, E, v);
  }
  const int ranks[1] = {n - k};
  SelTarget t[1];
  select_targets<NTH, 1, EM, MAXN>(v, n, base, E, ranks, sh, t);
  int eqb[2];
  sel_eq_before<NTH, 1, EM, MAXN>(v, E, cnt, t, sh, eqb);
  // selected = not below the cut
  int pos[3] = {0, 0, 0};
  {
    int eq = eqb[0];
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      if (j >= E) break;  // block-uniform
      eq += v[j] == t[0].prefix ? 1 : 0;
      pos[0] += (j < cnt && !sel_below(t[0], v[j], t[0].count - eq)) ? 1 : 0;
    }
  }
  int tot[3];
  block_exclusive_scan3(pos, tot, sh);
  int eq = eqb[0];
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    if (j >= E) break;  // block-uniform
    if (j < cnt) {
      eq += v[j] == t[0].prefix ? 1 : 0;
      if (!sel_below(t[0], v[j], t[0].count - eq)) {
        if (pos[0] < k) {  // an exact select never reaches the cap
          positions[pos[0]] = base + j;
          if (selected != nullptr) selected[pos[0]] = cv[j];
        }
        ++pos[0];
      }
    }
  }
}

// ---------------------------------------------------------------- linked top-k
// A packed 64-bit hand-over word: high half = tag | 0x80000000 (the valid
// bit), low half = payload bits; 0 means "not written yet".
__device__ __forceinline__ uint64_t pack_valid(uint32_t tag, uint32_t payload) {
  return ((uint64_t)(tag | 0x80000000u) << 32) | payload;
}
__device__ __forceinline__ bool is_valid(uint64_t w) { return (w >> 63) != 0; }

// The candidate top-k of the single-launch batch-1 step, where the scores come
// from other workgroups of the same launch.  Candidate i's word cand[i] is
// pack_valid(bits of |z_i|, bits of z_i) once its row is done (0 before).  The
// workgroup polls the words it has not seen yet (coherent loads, at most
// poll_limit rounds) and counts each score, as it arrives, into a histogram of
// its 12 leading value bits, so the counting overlaps the candidate rows.
// Once all n are in, a scan finds the bin of the target rank n - k; a bin of
// at most kSelResolve keys is resolved directly (every key ranks itself
// against the bin), a larger one (many equal scores) by the general select.
// The selection is the same as topk_block's.  It publishes the cut rather
// than a list: candidate position p with score bits x is selected iff
//     x > v,  or  x == v and p <= tie_pos,
// written as pack_valid(v, tie_pos) into the n_copies words thr[0],
// thr[stride], ... (coherent; each reader polls one copy, so no single line is
// polled by every workgroup).  Then, when not NULL, it writes positions
// (ascending, into C) and selected (channels C[p]) of the k selected
// candidates with plain stores, and with pairs not NULL (polled words only),
// for the j-th selected candidate in position order, pairs[j] =
// pack_valid(C[p], bits of z_p) (coherent; a reader polls its pairs until
// valid, so nothing depends on the order in which the cut and the pairs
// become visible).  A round
// limit reached sets *err (coherent); the step goes on with score 0 for the
// missing candidates.
// With score not NULL the scores are complete in memory already (an earlier
// launch wrote them): they are read once, cand and poll_limit unused.
template <int NTH, int MAXN>
__device__ __forceinline__ void topk_threshold_linked(const uint64_t* __restrict__ cand, int n, int k, const int32_t* __restrict__ C,
                                      int32_t* __restrict__ positions, int32_t* __restrict__ selected,
                                      uint64_t* __restrict__ thr, int n_copies, int stride, SelShared<NTH, MAXN>& sh,
                                      int poll_limit, uint32_t* err, const float* __restrict__ score = nullptr,
                                      uint64_t* __restrict__ pairs = nullptr) {
  constexpr int EM = SelShared<NTH, MAXN>::kPerThread;
  static_assert(sel_slot(MAXN - 1) < kSelSlots, "keys handed over through the histogram buffers");
  constexpr int kBinShift = 31 - 12;  // 12 leading value bits: 4096 bins
  if (n <= 0 || k <= 0) return;
  k = min(k, n);
  const int tid = threadIdx.x;
  for (int i = tid; i < kSelSlots; i += NTH) sh.hA[i] = 0u;
  __syncthreads();
  // ---- the scores as they arrive (element tid + j * NTH)
  uint32_t vb[EM], zb[EM];  // value bits of |z|, bits of z
  bool got[EM];
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    vb[j] = 0u;
    zb[j] = 0u;
    got[j] = tid + j * NTH >= n;
  }
  // bin of key u: (u - blo) >> bsh.  Polled words: the 12 leading value bits
  // (the range is not known in advance).  Scores in memory: 4096 bins over
  // their own [min, max], so that a bin rarely holds more than kSelResolve keys
  // even when the scores crowd into a few binades (maxima over a batch).
  uint32_t blo = 0u;
  int bsh = kBinShift;
  if (score != nullptr) {  // block-uniform
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < EM; ++j)
      if (!got[j]) {
        vb[j] = value_bits(score[tid + j * NTH]);
        mn = min(mn, vb[j]);
        mx = max(mx, vb[j]);
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    }
    if ((tid & 63) == 0) {
      sh.red[tid >> 6][0] = mn;
      sh.red[tid >> 6][1] = mx;
    }
    __syncthreads();
    mn = 0xffffffffu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
      mn = min(mn, sh.red[w][0]);
      mx = max(mx, sh.red[w][1]);
    }
    const uint32_t span = mx - mn;  // n >= 1: mn <= mx
    blo = mn;
    bsh = span < (uint32_t)kSelBins ? 0 : 32 - __builtin_clz(span) - 12;
#pragma unroll
    for (int j = 0; j < EM; ++j)
      if (!got[j]) {
        got[j] = true;
        atomicAdd(&sh.hA[sel_slot((int)((vb[j] - blo) >> bsh))], 1u);
      }
    __syncthreads();
  }
  for (int round = 0; score == nullptr; ++round) {
    // every word of the round is requested before any is examined (one
    // round trip a round; words already seen, and slots past n, read a valid
    // word again and are ignored)
    uint64_t wv[EM];
#pragma unroll
    for (int j = 0; j < EM; ++j)
      if (j * NTH < n) wv[j] = ld_coh(&cand[min(tid + j * NTH, n - 1)]);  // block-uniform condition
    bool all = true;
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      if (j * NTH < n && !got[j] && is_valid(wv[j])) {
        got[j] = true;
        vb[j] = (uint32_t)(wv[j] >> 32) & 0x7fffffffu;
        zb[j] = (uint32_t)wv[j];
        atomicAdd(&sh.hA[sel_slot((int)((vb[j] - blo) >> bsh))], 1u);
      }
      all &= got[j];
    }
    if (__syncthreads_and(all ? 1 : 0)) break;
    if (round + 1 >= poll_limit) {
      if (tid == 0) st_coh(err, 1u);
      // missing scores count as 0
#pragma unroll
      for (int j = 0; j < EM; ++j)
        if (!got[j]) {
          got[j] = true;
          atomicAdd(&sh.hA[sel_slot(0)], 1u);
        }
      __syncthreads();
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // ---- the bin holding ascending rank r = n - k
  constexpr int BPT = kSelBins / NTH;
  const int r = n - k;
  {
    unsigned int hb[BPT];
    int local = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      hb[b] = sh.hA[sel_slot(tid * BPT + b)];
      local += (int)hb[b];
    }
    int total;
    const int excl = block_excl_scan1(local, total, sh);
    if (r >= excl && r < excl + local) {
      int cum = excl;
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int c = (int)hb[b];
        if (r >= cum && r < cum + c) {
          SelTarget u;
          u.prefix = (uint32_t)(tid * BPT + b);  // the bin
          u.shift = bsh;
          u.rank = r - cum;
          u.count = c;
          u.beyond = 0;
          sh.tgt[0] = u;
        }
        cum += c;
      }
    }
  }
  __syncthreads();
  SelTarget t0 = sh.tgt[0];
  int tie_pos;
  bool published = false;
  if (t0.count <= kSelResolve) {
    // ---- small bin: gather its keys and rank each against the others
    if (tid == 0) sh.rcnt = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      const int i = tid + j * NTH;
      if (i < n && ((vb[j] - blo) >> bsh) == t0.prefix) {
        const int slot = atomicAdd(&sh.rcnt, 1);
        if (slot < kSelResolve) {
          sh.rv[slot] = vb[j];
          sh.ri[slot] = i;
        }
      }
    }
    __syncthreads();
    // Wave 0 ranks the bin's keys from registers (lane l holds key l): in
    // ascending order (smaller value first, on equal values the larger index
    // first) the key with t0.rank bin keys before it is the key of global
    // rank r, and the cut is that key's own (value, index): the selected
    // keys are those after it in this order, i.e. of larger value, or of
    // equal value and an index up to its own.  The wave publishes the cut
    // at once, with no block barrier in between.
    const int mb = t0.count;
    if (tid < 64) {
      const uint32_t vv = tid < mb ? sh.rv[tid] : 0xffffffffu;
      const int ii = tid < mb ? sh.ri[tid] : -1;
      int below = 0;
      for (int e = 0; e < mb; ++e) {
        const uint32_t ve = (uint32_t)__builtin_amdgcn_readlane((int)vv, e);
        const int ie = __builtin_amdgcn_readlane(ii, e);
        below += (ve < vv || (ve == vv && ie > ii)) ? 1 : 0;
      }
      const uint64_t hit = __ballot(tid < mb && below == t0.rank);
      const int src = hit != 0 ? (int)__builtin_ctzll(hit) : 0;
      const uint32_t cv = (uint32_t)__builtin_amdgcn_readlane((int)vv, src);
      const int tie = __builtin_amdgcn_readlane(ii, src);
      for (int c = tid; c < n_copies; c += 64) st_coh(&thr[c * stride], pack_valid(cv, (uint32_t)tie));
      if (tid == 0) {
        sh.tgt[1].prefix = cv;
        sh.scan[0][0] = tie;
      }
    }
    published = true;
    __syncthreads();
    t0.prefix = sh.tgt[1].prefix;
    tie_pos = sh.scan[0][0];
  } else {
    // ---- large bin: the general select over every key (owner layout)
    const int E = (n + NTH - 1) / NTH;
    const int base = tid * E;
    const int cnt = max(0, min(E, n - base));
#pragma unroll
    for (int j = 0; j < EM; ++j) {
      const int i = tid + j * NTH;
      if (i < n) sh.hB[sel_slot(i)] = vb[j];
    }
    __syncthreads();
    uint32_t v[EM];
#pragma unroll
    for (int j = 0; j < EM; ++j) v[j] = sh.hB[sel_slot(min(base + j, n - 1))];
    __syncthreads();  // the select clears the buffers next
    const int ranks[1] = {r};
    SelTarget t[1];
    select_targets<NTH, 1, EM, MAXN>(v, n, base, E, ranks, sh, t);
    int eqb[2];
    sel_eq_before<NTH, 1, EM, MAXN>(v, E, cnt, t, sh, eqb);
    const int m = t[0].count, q = t[0].rank;
    if (tid == 0) sh.scan[0][0] = q == 0 ? n : -1;
    __syncthreads();
    if (q > 0 && q < m) {
      int eq = eqb[0];
#pragma unroll
      for (int j = 0; j < EM; ++j) {
        if (j >= E) break;  // block-uniform
        if (j < cnt && v[j] == t[0].prefix) {
          ++eq;
          if (eq == m - q) sh.scan[0][0] = base + j;
        }
      }
    }
    __syncthreads();
    tie_pos = sh.scan[0][0];
    t0 = t[0];
  }
  const uint32_t cv = t0.prefix;
  if (!published && tid < n_copies) st_coh(&thr[tid * stride], pack_valid(cv, (uint32_t)tie_pos));
  if (positions == nullptr && selected == nullptr && pairs == nullptr) return;
  // ---- the list, ascending: flags (and with pairs, z) in LDS, then owner-layout scan
  __syncthreads();  // sh.scan and the LDS buffers are reused below
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    const int i = tid + j * NTH;
    if (i < n) {
      sh.hB[sel_slot(i)] = (vb[j] > cv || (vb[j] == cv && i <= tie_pos)) ? 1u : 0u;
      if (pairs != nullptr) sh.hA[sel_slot(i)] = zb[j];
    }
  }
  __syncthreads();
  const int E = (n + NTH - 1) / NTH;
  const int base = tid * E;
  const int cnt = max(0, min(E, n - base));
  int pos[3] = {0, 0, 0};
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    if (j >= E) break;  // block-uniform
    pos[0] += (j < cnt && sh.hB[sel_slot(base + j)] != 0u) ? 1 : 0;
  }
  int tot[3];
  block_exclusive_scan3(pos, tot, sh);
#pragma unroll
  for (int j = 0; j < EM; ++j) {
    if (j >= E) break;  // block-uniform
    if (j < cnt && sh.hB[sel_slot(base + j)] != 0u) {
      if (pos[0] < k) {
        if (positions != nullptr) positions[pos[0]] = base + j;
        if (selected != nullptr) selected[pos[0]] = C[base + j];
        if (pairs != nullptr) st_coh(&pairs[pos[0]], pack_valid((uint32_t)C[base + j], sh.hA[sel_slot(base + j)]));
      }
      ++pos[0];
    }
  }
}

// ---------------------------------------------------------------- fixed-order chunk sum
// out[i] = sum_{c < n_chunks} partial[c * n_out + i].  A block of 1024 threads
// covers 32 outputs; the chunks are dealt to 32 groups as contiguous ranges,
// each group sums its range in chunk order (8 loads in flight), and the 32
// group sums are added in group order: the same bits on every run.
template <int kUnused = 0>
__global__ __launch_bounds__(1024) void k_sum_chunks(const float* __restrict__ partial, int n_chunks, int64_t n_out,
                                                     float* __restrict__ out, unsigned int* __restrict__ reset,
                                                     int n_reset) {
  // Control words of the call's earlier kernels, cleared for the next call.
  if (reset != nullptr && blockIdx.x == 0 && (int)threadIdx.x < n_reset) reset[threadIdx.x] = 0u;
  __shared__ float part[32][33];
  const int o = threadIdx.x & 31;
  const int g = threadIdx.x >> 5;
  const int64_t i = (int64_t)blockIdx.x * 32 + o;
  const int per = (n_chunks + 31) / 32;
  const int c0 = g * per;
  const int c1 = min(n_chunks, c0 + per);
  float s = 0.f;
  if (i < n_out) {
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      float a[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = partial[(int64_t)(c + j) * n_out + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += a[j];
    }
    for (; c < c1; ++c) s += partial[(int64_t)c * n_out + i];
  }
  part[g][o] = s;
  __syncthreads();
  if (g == 0 && i < n_out) {
    float t = part[0][o];
#pragma unroll
    for (int j = 1; j < 32; ++j) t += part[j][o];
    out[i] = t;
  }
}

// out[i] = sum_{c < n_chunks} partial[c * n_out + i] in chunk order, one
// thread per output with all n_chunks <= MAXC loads in flight at once (padded
// loads re-read the last chunk and add nothing): for the few dozen chunks of
// the matrix-core down-projection, where the grouped sum above would leave
// most of its threads idle.
// reset / n_reset / reset_stride: hand-over words of the launch before
// (reset[t * reset_stride], t < n_reset) cleared for the next call.
template <int MAXC>
__global__ __launch_bounds__(256) void k_sum_few(const float* __restrict__ partial, int n_chunks, int64_t n_out,
                                                 float* __restrict__ out, uint64_t* reset, int n_reset,
                                                 int reset_stride) {
  if (blockIdx.x == 0 && (int)threadIdx.x < n_reset) st_coh(&reset[(int64_t)threadIdx.x * reset_stride], (uint64_t)0);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_out) return;
  float a[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) a[c] = partial[(int64_t)min(c, n_chunks - 1) * n_out + i];
  float s = a[0];
#pragma unroll
  for (int c = 1; c < MAXC; ++c)
    if (c < n_chunks) s += a[c];
  out[i] = s;
}

}  // namespace pop
