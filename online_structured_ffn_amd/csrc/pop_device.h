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
// unique.  For each of NT targets (ascending ranks) the select finds a
// threshold such that  less(key)  holds exactly for the c keys below rank c.
//
// The value bits sit in LDS (sh.vals).  Thread t owns the consecutive elements
// [t*E, min(n, (t+1)*E)), E = ceil(n / kSelThreads).  The radix passes start at
// the highest bit where the values differ (all common leading bits are
// skipped, so the first pass spreads over the histogram), use 8-bit digits and
// stop for a target as soon as its bucket holds a single key.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelMaxN = 32768;

struct SelTarget {
  unsigned long long prefix;  // key bits at positions >= known
  int known;                  // lowest known bit position
  int rank;                   // remaining rank inside the current bucket
  int state;                  // 0 active, 1 found, 2 rank >= n (every key is below)
};

struct SelShared {
  uint32_t vals[kSelMaxN];
  unsigned int hist[2][256];
  SelTarget tgt[2];
  unsigned int red_or[16];
  unsigned int red_and[16];
  int scan[16][3];
};

__device__ __forceinline__ unsigned long long sel_key(uint32_t vb, int i) {
  return ((unsigned long long)vb << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

__device__ __forceinline__ bool sel_less(const SelTarget& t, unsigned long long key) {
  if (t.state == 2) return true;
  return (key >> t.known) < (t.prefix >> t.known);
}

// Loads value_bits of src[0..n) into sh.vals (all threads), then a barrier.
__device__ __forceinline__ void sel_load(const float* __restrict__ src, int n, SelShared& sh) {
  for (int i = threadIdx.x; i < n; i += kSelThreads) sh.vals[i] = value_bits(src[i]);
  __syncthreads();
}

template <int NT>
__device__ void select_thresholds(int n, const int (&ranks)[NT], SelShared& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = (n + kSelThreads - 1) / kSelThreads;
  const int base = tid * E;
  const int end = min(n, base + E);

  // Common leading bits of every value.
  uint32_t vor = 0u, vand = 0xffffffffu;
  for (int i = base; i < end; ++i) {
    vor |= sh.vals[i];
    vand &= sh.vals[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    vor |= __shfl_xor(vor, o);
    vand &= __shfl_xor(vand, o);
  }
  if (lane == 0) {
    sh.red_or[wave] = vor;
    sh.red_and[wave] = vand;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t a = 0u, b = 0xffffffffu;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      a |= sh.red_or[w];
      b &= sh.red_and[w];
    }
    const uint32_t diff = a ^ b;
    int top;  // highest key bit that can differ
    unsigned long long prefix;
    if (n == 0) {
      top = 31;
      prefix = 0ull;
    } else if (diff == 0u) {
      top = 31;  // every value equal: only the index half differs
      prefix = (unsigned long long)b << 32;
    } else {
      const int hb = 31 - __clz(diff);
      top = 32 + hb;
      const uint32_t keep = (hb == 31) ? 0u : ~((2u << hb) - 1u);
      prefix = (unsigned long long)(b & keep) << 32;
    }
    for (int t = 0; t < NT; ++t) {
      sh.tgt[t].prefix = prefix;
      sh.tgt[t].known = top + 1;
      sh.tgt[t].rank = ranks[t];
      sh.tgt[t].state = (ranks[t] >= n) ? 2 : 0;
    }
  }
  __syncthreads();

  // At most 8 passes per target: 63 key bits in 8-bit digits.
  for (int pass = 0; pass < 16; ++pass) {
    bool active = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) active |= (sh.tgt[t].state == 0);
    if (!active) break;  // uniform: every thread reads the same shared state

    for (int i = tid; i < NT * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0u;
    __syncthreads();

#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const SelTarget tg = sh.tgt[t];
      if (tg.state != 0) continue;
      const int s = tg.known > 8 ? tg.known - 8 : 0;
      const unsigned long long mask = (1ull << (tg.known - s)) - 1ull;
      for (int i = base; i < end; ++i) {
        const unsigned long long key = sel_key(sh.vals[i], i);
        if (((key ^ tg.prefix) >> tg.known) == 0ull) atomicAdd(&sh.hist[t][(int)((key >> s) & mask)], 1u);
      }
    }
    __syncthreads();

    if (wave < NT) {
      const int t = wave;
      const SelTarget tg = sh.tgt[t];
      if (tg.state == 0) {
        const int s = tg.known > 8 ? tg.known - 8 : 0;
        unsigned int c[4];
        unsigned int sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = sh.hist[t][lane * 4 + j];
          sum += c[j];
        }
        unsigned int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned int v = __shfl_up(incl, o);
          if (lane >= o) incl += v;
        }
        unsigned int before = incl - sum;
        const unsigned int rk = (unsigned int)tg.rank;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (c[j] > 0u && before <= rk && rk < before + c[j]) {
            SelTarget nt;
            nt.prefix = tg.prefix | ((unsigned long long)(lane * 4 + j) << s);
            nt.known = s;
            nt.rank = (int)(rk - before);
            nt.state = (c[j] == 1u || s == 0) ? 1 : 0;
            sh.tgt[t] = nt;
          }
          before += c[j];
        }
      }
    }
    __syncthreads();
  }
}

// Block-wide exclusive scan of up to three per-thread counters (1024 threads).
__device__ __forceinline__ void block_exclusive_scan3(int (&v)[3], int (&total)[3], SelShared& sh) {
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
    for (int w = 0; w < kSelThreads / 64; ++w) {
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

// ---------------------------------------------------------------- fixed-order chunk sum
// out[i] = sum_{c < n_chunks} partial[c * n_out + i], summed as 8 contiguous
// groups of chunks (each in chunk order) then the 8 group sums in group order:
// the same bits on every run.
template <int kUnused = 0>
__global__ __launch_bounds__(256) void k_sum_chunks(const float* __restrict__ partial, int n_chunks, int64_t n_out,
                                                    float* __restrict__ out) {
  __shared__ float part[8][33];
  const int o = threadIdx.x & 31;
  const int g = threadIdx.x >> 5;
  const int64_t i = (int64_t)blockIdx.x * 32 + o;
  const int per = (n_chunks + 7) / 8;
  const int c0 = g * per;
  const int c1 = min(n_chunks, c0 + per);
  float s = 0.f;
  if (i < n_out) {
    int c = c0;
    for (; c + 4 <= c1; c += 4) {
      const float a0 = partial[(int64_t)c * n_out + i];
      const float a1 = partial[(int64_t)(c + 1) * n_out + i];
      const float a2 = partial[(int64_t)(c + 2) * n_out + i];
      const float a3 = partial[(int64_t)(c + 3) * n_out + i];
      s += a0;
      s += a1;
      s += a2;
      s += a3;
    }
    for (; c < c1; ++c) s += partial[(int64_t)c * n_out + i];
  }
  part[g][o] = s;
  __syncthreads();
  if (g == 0 && i < n_out) {
    float t = part[0][o];
#pragma unroll
    for (int j = 1; j < 8; ++j) t += part[j][o];
    out[i] = t;
  }
}

}  // namespace pop
