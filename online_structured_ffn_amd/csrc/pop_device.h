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
// One-workgroup exact selection over n <= kSelMaxN keys.
//
// Element i (0 <= i < n) has the 64-bit key  (value_bits << 32) | (0xffffffff - i):
// a larger value is more important and, on equal values, the lower index is
// more important.  All keys are distinct, so "the key of ascending rank c" is
// unique.  For each of NT targets (ascending ranks) the select finds the key T
// of that rank; less(key) := key < T then holds for exactly c keys.
//
// The value bits sit in LDS (sh.vals).  Thread t owns the consecutive elements
// [t*E, min(n, (t+1)*E)), E = ceil(n / NTH).
//   pass 1   an 11-bit digit taken just below the common leading bits of all n
//            keys (so the digit always splits the set), one 2048-bin histogram
//            and a block scan locate each target's bucket;
//   compact  a bucket of at most kSelListCap keys is copied to a list, so later
//            passes scan only the bucket;
//   passes   8-bit digits below the known bits until a bucket holds at most
//            kSelBrute keys;
//   rank     the last bucket's keys are copied to LDS and ranked by direct
//            comparison (one thread per key, the comparisons' LDS reads
//            independent of each other), and the key of the target rank
//            becomes the threshold.
// Every loop is bounded; every LDS write index is checked against its array.
// ---------------------------------------------------------------------------
constexpr int kSelMaxN = 32768;
constexpr int kSelBins1 = 2048;
constexpr int kSelListCap = 2048;
constexpr int kSelBrute = 32;

struct SelTarget {
  unsigned long long prefix;  // key bits at positions >= known (the whole key once state == 1)
  int known;                  // lowest known bit position (0 once state == 1)
  int rank;                   // remaining rank inside the current bucket
  int count;                  // keys in the current bucket
  int state;                  // 0 searching, 1 found, 2 rank >= n (every key is below)
};

template <int NTH, int MAXN = kSelMaxN>
struct SelShared {
  uint32_t vals[MAXN];
  unsigned int hist[kSelBins1];
  int list[2][kSelListCap];
  unsigned long long skey[2][kSelBrute];
  int list_n[2];   // -1: the bucket is scanned in the full array
  int small_n[2];
  SelTarget tgt[2];
  uint32_t red[NTH / 64][4];
  int scan[NTH / 64][3];
};

__device__ __forceinline__ unsigned long long sel_key(uint32_t vb, int i) {
  return ((unsigned long long)vb << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

__device__ __forceinline__ bool sel_less(const SelTarget& t, unsigned long long key) {
  if (t.state == 2) return true;
  return (key >> t.known) < (t.prefix >> t.known);
}

__device__ __forceinline__ bool sel_in_bucket(const SelTarget& t, unsigned long long key) {
  return t.known >= 64 || ((key ^ t.prefix) >> t.known) == 0ull;
}

// Loads value_bits of src[0..n) into sh.vals, then a barrier.
template <int NTH, int MAXN>
__device__ __forceinline__ void sel_load(const float* __restrict__ src, int n, SelShared<NTH, MAXN>& sh) {
  // 8 loads in flight per thread before any LDS store.
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * NTH) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (i0 + j * NTH < n) ? src[i0 + j * NTH] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (i0 + j * NTH < n) sh.vals[i0 + j * NTH] = value_bits(v[j]);
  }
  __syncthreads();
}

// Block-wide exclusive scan of one int per thread; returns the exclusive
// prefix and (through total) the block sum.  Contains two barriers.
template <int NTH, int MAXN>
__device__ __forceinline__ int block_excl_scan1(int v, int& total, SelShared<NTH, MAXN>& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh.scan[wave][0] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const int x = sh.scan[w][0];
    off += (w < wave) ? x : 0;
    tot += x;
  }
  total = tot;
  __syncthreads();
  return off + incl - v;
}

template <int NTH, int NT, int MAXN>
__device__ void select_thresholds(int n, const int (&ranks)[NT], SelShared<NTH, MAXN>& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = (n + NTH - 1) / NTH;
  const int base = tid * E;
  const int end = min(n, base + E);

  // ---- A. common leading bits of all keys
  uint32_t hor = 0u, hand = 0xffffffffu, lor = 0u, land = 0xffffffffu;
  for (int i = base; i < end; ++i) {
    const uint32_t v = sh.vals[i];
    const uint32_t lo = 0xffffffffu - (uint32_t)i;
    hor |= v;
    hand &= v;
    lor |= lo;
    land &= lo;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    hor |= __shfl_xor(hor, o);
    hand &= __shfl_xor(hand, o);
    lor |= __shfl_xor(lor, o);
    land &= __shfl_xor(land, o);
  }
  if (lane == 0) {
    sh.red[wave][0] = hor;
    sh.red[wave][1] = hand;
    sh.red[wave][2] = lor;
    sh.red[wave][3] = land;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t a0 = 0u, b0 = 0xffffffffu, a1 = 0u, b1 = 0xffffffffu;
    for (int w = 0; w < NTH / 64; ++w) {
      a0 |= sh.red[w][0];
      b0 &= sh.red[w][1];
      a1 |= sh.red[w][2];
      b1 &= sh.red[w][3];
    }
    const unsigned long long kor = ((unsigned long long)a0 << 32) | a1;
    const unsigned long long kand = ((unsigned long long)b0 << 32) | b1;
    const unsigned long long diff = kor ^ kand;
    const int known = diff ? 64 - __clzll(diff) : 0;  // bits >= known are common to all keys
    const unsigned long long prefix = known >= 64 ? 0ull : (kand >> known) << known;
    for (int t = 0; t < NT; ++t) {
      SelTarget g;
      g.prefix = prefix;
      g.known = known;
      g.rank = ranks[t];
      g.count = n;
      g.state = ranks[t] >= n ? 2 : (n == 1 ? 1 : 0);
      if (g.state == 1) {  // a single key: it is the threshold
        g.prefix = kand;
        g.known = 0;
      }
      sh.tgt[t] = g;
      sh.list_n[t] = -1;
    }
  }
  __syncthreads();

  // ---- B. first pass: 11-bit digit just below the common bits
  bool any = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) any |= sh.tgt[t].state == 0;
  if (any) {
    const int known0 = sh.tgt[0].known;  // every target starts from the same common bits
    const int s1 = known0 > 11 ? known0 - 11 : 0;
    const unsigned long long mask1 = (1ull << (known0 - s1)) - 1ull;
    for (int i = tid; i < kSelBins1; i += NTH) sh.hist[i] = 0u;
    __syncthreads();
    for (int i = base; i < end; ++i)
      atomicAdd(&sh.hist[(int)((sel_key(sh.vals[i], i) >> s1) & mask1)], 1u);
    __syncthreads();
    constexpr int BPT = kSelBins1 / NTH;  // bins per thread
    unsigned int c[BPT];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = sh.hist[tid * BPT + j];
      sum += (int)c[j];
    }
    // Snapshot the targets before the scan: its barriers order every read
    // here before the single write per target below.
    SelTarget snap[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) snap[t] = sh.tgt[t];
    int total;
    const int before0 = block_excl_scan1(sum, total, sh);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const SelTarget g = snap[t];
      if (g.state != 0) continue;
      int before = before0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        if (c[j] > 0u && before <= g.rank && g.rank < before + (int)c[j]) {
          SelTarget h = g;
          h.prefix = g.prefix | ((unsigned long long)(tid * BPT + j) << s1);
          h.known = s1;
          h.rank = g.rank - before;
          h.count = (int)c[j];
          sh.tgt[t] = h;
        }
        before += (int)c[j];
      }
    }
    __syncthreads();
    // compact small-enough buckets into lists
    if (tid < NT) sh.list_n[tid] = (sh.tgt[tid].state == 0 && sh.tgt[tid].count <= kSelListCap) ? 0 : -1;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const SelTarget g = sh.tgt[t];
      if (g.state != 0 || sh.list_n[t] < 0) continue;
      for (int i = base; i < end; ++i) {
        if (sel_in_bucket(g, sel_key(sh.vals[i], i))) {
          const int pos = atomicAdd(&sh.list_n[t], 1);
          if (pos < kSelListCap) sh.list[t][pos] = i;
        }
      }
    }
    __syncthreads();
  }

  // ---- C. 8-bit passes until every bucket is small, then rank directly
  for (int pass = 0; pass < 16; ++pass) {
    bool big = false, active = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      active |= sh.tgt[t].state == 0;
      big |= sh.tgt[t].state == 0 && sh.tgt[t].count > kSelBrute;
    }
    if (!active) break;
    if (big) {
      for (int i = tid; i < NT * 256; i += NTH) sh.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const SelTarget g = sh.tgt[t];
        if (g.state != 0 || g.count <= kSelBrute) continue;
        const int s = g.known > 8 ? g.known - 8 : 0;
        const unsigned long long mask = (1ull << (g.known - s)) - 1ull;
        const int ln = sh.list_n[t];
        if (ln >= 0) {
          for (int j = tid; j < ln && j < kSelListCap; j += NTH) {
            const int i = sh.list[t][j];
            const unsigned long long key = sel_key(sh.vals[i], i);
            if (sel_in_bucket(g, key)) atomicAdd(&sh.hist[t * 256 + (int)((key >> s) & mask)], 1u);
          }
        } else {
          for (int i = base; i < end; ++i) {
            const unsigned long long key = sel_key(sh.vals[i], i);
            if (sel_in_bucket(g, key)) atomicAdd(&sh.hist[t * 256 + (int)((key >> s) & mask)], 1u);
          }
        }
      }
      __syncthreads();
      if (wave < NT) {
        const int t = wave;
        const SelTarget g = sh.tgt[t];
        if (g.state == 0 && g.count > kSelBrute) {
          const int s = g.known > 8 ? g.known - 8 : 0;
          unsigned int cc[4];
          unsigned int sum = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            cc[j] = sh.hist[t * 256 + lane * 4 + j];
            sum += cc[j];
          }
          unsigned int incl = sum;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const unsigned int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
          }
          unsigned int before = incl - sum;
          const unsigned int rk = (unsigned int)g.rank;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (cc[j] > 0u && before <= rk && rk < before + cc[j]) {
              SelTarget h = g;
              h.prefix = g.prefix | ((unsigned long long)(lane * 4 + j) << s);
              h.known = s;
              h.rank = (int)(rk - before);
              h.count = (int)cc[j];
              sh.tgt[t] = h;
            }
            before += cc[j];
          }
        }
      }
      __syncthreads();
      continue;
    }
    // every active bucket holds at most kSelBrute keys: gather and rank them
    if (tid < NT) sh.small_n[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const SelTarget g = sh.tgt[t];
      if (g.state != 0) continue;
      const int ln = sh.list_n[t];
      if (ln >= 0) {
        for (int j = tid; j < ln && j < kSelListCap; j += NTH) {
          const int i = sh.list[t][j];
          const unsigned long long key = sel_key(sh.vals[i], i);
          if (sel_in_bucket(g, key)) {
            const int pos = atomicAdd(&sh.small_n[t], 1);
            if (pos < kSelBrute) sh.skey[t][pos] = key;
          }
        }
      } else {
        for (int i = base; i < end; ++i) {
          const unsigned long long key = sel_key(sh.vals[i], i);
          if (sel_in_bucket(g, key)) {
            const int pos = atomicAdd(&sh.small_n[t], 1);
            if (pos < kSelBrute) sh.skey[t][pos] = key;
          }
        }
      }
    }
    __syncthreads();
    SelTarget snap2[NT];
    int msnap[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      snap2[t] = sh.tgt[t];
      msnap[t] = min(sh.small_n[t], kSelBrute);
    }
    __syncthreads();  // every thread holds its snapshot before any target is rewritten
    for (int slot = tid; slot < NT * kSelBrute; slot += NTH) {
      const int t = slot / kSelBrute;
      const int j = slot % kSelBrute;
      const SelTarget g = (t == 0) ? snap2[0] : snap2[NT - 1];  // no runtime-indexed register array
      const int m = (t == 0) ? msnap[0] : msnap[NT - 1];
      if (g.state != 0 || j >= m) continue;
      const unsigned long long kj = sh.skey[t][j];
      int r = 0;
#pragma unroll 8
      for (int q = 0; q < kSelBrute; ++q) r += (q < m && sh.skey[t][q] < kj) ? 1 : 0;
      if (r == g.rank) {
        SelTarget h = g;
        h.prefix = kj;
        h.known = 0;
        h.rank = 0;
        h.count = 1;
        h.state = 1;
        sh.tgt[t] = h;
      }
    }
    __syncthreads();
    break;
  }
}

// Block-wide exclusive scan of three per-thread counters.
template <int NTH, int MAXN>
__device__ __forceinline__ void block_exclusive_scan3(int (&v)[3], int (&total)[3], SelShared<NTH, MAXN>& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int incl[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    incl[j] = v[j];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl[j], o);
      if (lane >= o) incl[j] += u;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < 3; ++j) sh.scan[wave][j] = incl[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    int off = 0, tot = 0;
    for (int w = 0; w < NTH / 64; ++w) {
      const int x = sh.scan[w][j];
      if (w < wave) off += x;
      tot += x;
    }
    const int excl = off + incl[j] - v[j];
    v[j] = excl;
    total[j] = tot;
  }
  __syncthreads();
}

// S = the k most important of n candidates (score descending, position
// ascending on ties), written in ascending order as positions into C and, when
// `selected` is not NULL, as channels C[position].  One workgroup.
template <int NTH, int MAXN>
__device__ void topk_block(const float* __restrict__ score, int n, int k, const int32_t* __restrict__ C,
                           int32_t* __restrict__ positions, int32_t* __restrict__ selected, SelShared<NTH, MAXN>& sh) {
  // For up to 16 keys per thread, this thread's channels C[base, end) are
  // fetched with the scores, so the final write waits on no further global
  // load; wider launches read them at the end.
  constexpr int EM = (MAXN + NTH - 1) / NTH;
  constexpr int EP = EM <= 16 ? EM : 1;
  const int E = (n + NTH - 1) / NTH;
  const int base = threadIdx.x * E;
  const int end = min(n, base + E);
  int cv[EP];
  if (EM <= 16 && selected != nullptr) {
#pragma unroll
    for (int j = 0; j < EP; ++j) cv[j] = C[max(0, min(base + j, n - 1))];
  }
  sel_load(score, n, sh);
  const int ranks[1] = {n - k};
  select_thresholds(n, ranks, sh);
  const SelTarget t = sh.tgt[0];
  int pos[3] = {0, 0, 0};
  for (int i = base; i < end; ++i)
    if (!sel_less(t, sel_key(sh.vals[i], i))) ++pos[0];
  int tot[3];
  block_exclusive_scan3(pos, tot, sh);
  if constexpr (EM <= 16) {
#pragma unroll
    for (int j = 0; j < EP; ++j) {
      const int i = base + j;
      if (i < end && !sel_less(t, sel_key(sh.vals[i], i))) {
        if (pos[0] < k) {  // an exact select never reaches the cap
          positions[pos[0]] = i;
          if (selected != nullptr) selected[pos[0]] = cv[j];
        }
        ++pos[0];
      }
    }
  } else {
    for (int i = base; i < end; ++i) {
      if (!sel_less(t, sel_key(sh.vals[i], i))) {
        if (pos[0] < k) {
          positions[pos[0]] = i;
          if (selected != nullptr) selected[pos[0]] = C[i];
        }
        ++pos[0];
      }
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

}  // namespace pop
