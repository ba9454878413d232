// Batched decode (B >= 2 rows share one mask) on the matrix cores, bf16.
//
// At batch B the gate/up stage is a skinny product Z = x W^T over the rows of
// R u C (M = B tokens, N = |R u C|, K = d) and the down stage is
// Y = Z W_downT over the live rows (M = B, N = d, K = |R| + k): both are
// HBM-bound (B flops per weight byte) but far too instruction-heavy for plain
// FMA loops once B reaches ~8.  Here both run as v_mfma_f32_16x16x32_bf16 with
// the tokens as the M dimension (16 per tile, up to kDecMaxTiles tiles).
//
// Fragment layout of the 16x16x32 product (lane l of a wave): A row l & 15,
// B column l & 15, each with the 8 consecutive reduction indices
// 8 (l >> 4) + [0, 8); accumulator element e is row 4 (l >> 4) + e, column
// l & 15.  One load instruction thus reads 64 contiguous bytes of each of 16
// rows.
#pragma once
#include <hip/hip_runtime.h>

#include "pop_device.h"

namespace pop {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecMaxTiles = 4;  // up to 64 tokens on the matrix cores

__device__ __forceinline__ int clamp_ch(int ch, int d_ff) { return min(max(ch, 0), d_ff - 1); }

__device__ __forceinline__ f32x4_t mfma16(u32x4 a, u32x4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_pack_rne(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a += 0x7fffu + ((a >> 16) & 1u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xffff0000u);
}

// ---------------------------------------------------------------- gate / up
// Block b: rows p0 = 16 NT b + [0, 16 NT) of R u C (identity rows with
// kIdentity) in NT tiles of 16 that share the token fragments, every token.
// Wave w reduces over k in [w * kq, (w + 1) * kq), kq a multiple of 64; the
// four partial products meet in LDS, then z = SiLU(g) * u is written for every
// (token, row) and, for candidate rows, the score max over tokens of |z|.
#ifndef POP_GU_NT
#define POP_GU_NT 1
#endif
constexpr int kGuNT = POP_GU_NT;  // row tiles per block

template <int MT, bool kIdentity>
__global__ __launch_bounds__(256) void k_gateup_mfma(const bf16s* __restrict__ x, int B, int d,
                                                     const bf16s* __restrict__ Wg, const bf16s* __restrict__ Wu,
                                                     int d_ff, const int32_t* __restrict__ R, int n_R,
                                                     const int32_t* __restrict__ C, int n_C, float* __restrict__ z,
                                                     float* __restrict__ score) {
  constexpr int NT = kGuNT;
  __shared__ f32x4_t red[3][2 * MT * NT][64];
  // The wave index as a scalar: the K range and every loop condition below
  // are then uniform branches, not exec-mask regions.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int n_A = n_R + n_C;
  const int p0 = blockIdx.x * 16 * NT;
  // this lane's weight rows (rows past n_A repeat the last one; never stored)
  const bf16s* wg[NT];
  const bf16s* wu[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int p = min(p0 + 16 * n + r, n_A - 1);
    const int ch = kIdentity ? p : clamp_ch(p < n_R ? R[p] : C[p - n_R], d_ff);
    wg[n] = Wg + (int64_t)ch * d;
    wu[n] = Wu + (int64_t)ch * d;
  }
  // this lane's token rows of x
  const bf16s* xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tok = 16 * t + r;
    xr[t] = x + (int64_t)(tok < B ? tok : 0) * d;
  }
  const int kq = ((d + 255) / 256) * 64;  // per-wave share, a multiple of 64
  const int kb = wave * kq, ke = min(d, kb + kq);
  f32x4_t ag[NT][MT], au[NT][MT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int t = 0; t < MT; ++t) ag[n][t] = au[n][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // One 64-wide step: the lane's 16-byte vectors at k0 + 8 g and k0 + 32 + 8 g
  // of each gate and up row and of every token row; token vectors past ke are
  // zero (d % 8 == 0, so a vector is all in or all out) and the weight loads
  // stay in the row.
  // The buffers hold the raw loads; the zeroing of vectors past ke happens at
  // use, so no wait is forced between issuing a step's loads and using the
  // previous step's (the memory counter is in order: an early wait on the
  // newest load would drain the whole pipeline).  Tokens past B read token 0's
  // row: their products are never stored.
  struct Step {
    u32x4 g0[NT], g1[NT], u0[NT], u1[NT], xa[MT], xb[MT];
    bool on_a, on_b;
  };
  auto load = [&](Step& S, int k0, bool valid) {
    const int ka = k0 + 8 * g, kb8 = ka + 32;
    S.on_a = valid && ka < ke;
    S.on_b = valid && kb8 < ke;
    const int ca = S.on_a ? ka : 0, cb = S.on_b ? kb8 : 0;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      S.g0[n] = ld16(wg[n] + ca);  // plain loads measured faster than non-temporal here
      S.g1[n] = ld16(wg[n] + cb);
      S.u0[n] = ld16(wu[n] + ca);
      S.u1[n] = ld16(wu[n] + cb);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      S.xa[t] = ld16(xr[t] + ca);
      S.xb[t] = ld16(xr[t] + cb);
    }
  };
  auto use = [&](const Step& S) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4 xa = S.on_a ? S.xa[t] : zero, xb = S.on_b ? S.xb[t] : zero;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        ag[n][t] = mfma16(xa, S.g0[n], ag[n][t]);
        ag[n][t] = mfma16(xb, S.g1[n], ag[n][t]);
        au[n][t] = mfma16(xa, S.u0[n], au[n][t]);
        au[n][t] = mfma16(xb, S.u1[n], au[n][t]);
      }
    }
  };
  // A ring of DEPTH steps in flight.  The loop body has no branch: the step
  // count is padded to a multiple of DEPTH, steps past the last one re-read it
  // (cache hits) with their operands zeroed, and the scheduling barriers keep
  // each prefetch ahead of the products it hides.
  constexpr int DEPTH = MT <= 2 ? 4 : 2;
  const int nsteps = ke > kb ? (ke - kb + 63) / 64 : 0;
  const int last = nsteps > 0 ? nsteps - 1 : 0;
  auto kstep = [&](int st) { return kb + 64 * min(st, last); };
  Step S[DEPTH];
  if (nsteps > 0) {
#pragma unroll
    for (int j = 0; j < DEPTH - 1; ++j) load(S[j], kstep(j), j < nsteps);
    for (int st = 0; st < nsteps; st += DEPTH) {
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) {
        const int ahead = st + j + DEPTH - 1;
        load(S[(j + DEPTH - 1) % DEPTH], kstep(ahead), ahead < nsteps);
        __builtin_amdgcn_sched_barrier(0);
        use(S[j]);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        red[wave - 1][2 * (n * MT + t)][lane] = ag[n][t];
        red[wave - 1][2 * (n * MT + t) + 1][lane] = au[n][t];
      }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float smax = 0.f;
    const int prow = p0 + 16 * n + r;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      f32x4_t gs = ag[n][t], us = au[n][t];
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        gs += red[w][2 * (n * MT + t)][lane];
        us += red[w][2 * (n * MT + t) + 1][lane];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * t + 4 * g + e;
        if (tok < B) {
          const float zz = silu(gs[e]) * us[e];
          if (prow < n_A) z[(int64_t)tok * n_A + prow] = zz;
          smax = fmaxf(smax, fabsf(zz));
        }
      }
    }
    // max over the four lane groups (tokens) of the same row
    smax = fmaxf(smax, __shfl_xor(smax, 16));
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    if (g == 0 && prow >= n_R && prow < n_A && score != nullptr) score[prow - n_R] = smax;
  }
}

// ---------------------------------------------------------------- down
// zl[b][q] = bf16(z[b][column of live row q]) for q < n_live (R first, then the
// selected channels at n_R + pos), zero up to the row pitch ldl (a multiple of
// 8 at least one tile past n_live): the down-projection's A operand in live
// order, gathered once.
__global__ __launch_bounds__(256) void k_gather_zlive(const float* __restrict__ z, int n_A, int B, int n_R,
                                                      const int32_t* __restrict__ pos, int n_live, int ldl,
                                                      uint16_t* __restrict__ zl) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // a pair of columns
  const int q = 2 * (i % (ldl / 2)), b = i / (ldl / 2);
  if (b >= B) return;
  const float* zr = z + (int64_t)b * n_A;
  auto col = [&](int qq) { return qq < n_R ? qq : min(n_R + max(pos[qq - n_R], 0), n_A - 1); };
  const float a = q < n_live ? zr[col(q)] : 0.f;
  const float c = q + 1 < n_live ? zr[col(q + 1)] : 0.f;
  reinterpret_cast<uint32_t*>(zl + (int64_t)b * ldl)[q / 2] = bf16_pack_rne(a, c);
}

// Block (cs, c): output columns cs * 64 + [0, 64) over the live rows
// [c * rows_per_chunk, ...) (R first, then the selected channels; at most
// kDownMaxChunk rows, a multiple of 8).  Every W_downT load of the chunk is
// issued at once (the 128 contiguous bytes of each row); the rows then go to
// LDS transposed as (row, row + 1) pairs — thread t takes row pairs 32 i +
// (t & 31) at columns (t >> 5) * 8 + [0, 8), so a half-wave's 32 pairs cover
// all 64 banks.  The A operand comes straight from zl (16-byte vectors of 8
// live rows).  Wave w owns the 16 columns 16 w + [0, 16).  Writes
// partial[c][token][col].
constexpr int kDownMaxChunk = 256;                 // live rows per block
constexpr int kDownTileRows = kDownMaxChunk;        // padding of zl past n_live
constexpr int kDownLd = kDownMaxChunk + 8;         // Bt pitch in bf16 (528 bytes)
constexpr int kDownPairs = kDownMaxChunk / 64;     // row pairs per thread

template <int MT, bool kIdentity>
__global__ __launch_bounds__(256) void k_down_mfma(const uint16_t* __restrict__ zl, int ldl, int B,
                                                   const bf16s* __restrict__ WdT, int d, int d_ff,
                                                   const int32_t* __restrict__ R, int n_R,
                                                   const int32_t* __restrict__ sel, int n_live, int rows_per_chunk,
                                                   float* __restrict__ partial) {
  __shared__ __align__(16) uint16_t Bt[64 * kDownLd];  // [column][row of the chunk]
  __shared__ int rch[kDownMaxChunk];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * 64;
  const int q0 = blockIdx.y * rows_per_chunk;
  const int nrows = max(0, min(n_live, q0 + rows_per_chunk) - q0);
  // channel of every live row of the chunk
  for (int i = tid; i < kDownMaxChunk; i += 256) {
    int chv = 0;
    if (i < nrows) {
      const int q = q0 + i;
      chv = kIdentity ? q : clamp_ch(q < n_R ? R[q] : sel[q - n_R], d_ff);
    }
    rch[i] = chv;
  }
  __syncthreads();
  const int kp = tid & 31, cc = (tid >> 5) * 8;
  const bool col_on = c0 + cc < d;  // d % 8 == 0
  const int col_c = col_on ? c0 + cc : d - 8;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // every row pair of the chunk (clamped, unconditional loads; zeroed below)
  u32x4 va[kDownPairs], vb[kDownPairs];
#pragma unroll
  for (int h = 0; h < kDownPairs; ++h) {
    const int qa = 64 * h + 2 * kp;
    va[h] = ld16(WdT + (int64_t)rch[qa] * d + col_c);  // plain loads: measured faster than non-temporal
    vb[h] = ld16(WdT + (int64_t)rch[qa + 1] * d + col_c);
  }
  // the A fragments: tokens past B read token 0 (their sums are never
  // stored); q0 is a multiple of 8 and zl carries kDownTileRows rows of zero
  // padding past n_live, so the vectors are aligned and inside the row
  const uint16_t* zrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) zrow[t] = zl + (int64_t)min(16 * t + r, B - 1) * ldl + q0 + 8 * g;
  const int nk = (nrows + 31) / 32;  // 32-row product steps
  u32x4 fa[MT][kDownMaxChunk / 32];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int kk = 0; kk < kDownMaxChunk / 32; ++kk)
      fa[t][kk] = kk < nk ? *reinterpret_cast<const u32x4*>(zrow[t] + 32 * kk) : zero;
  uint32_t* b32 = reinterpret_cast<uint32_t*>(Bt);
#pragma unroll
  for (int h = 0; h < kDownPairs; ++h) {
    if (64 * h >= nrows) continue;  // rows past 32 * nk are never read
    const int qa = 64 * h + 2 * kp;
    const u32x4 ta = (col_on && qa < nrows) ? va[h] : zero;
    const u32x4 tb = (col_on && qa + 1 < nrows) ? vb[h] : zero;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = (ta[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
      const uint32_t hi = (tb[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
      b32[((cc + j) * kDownLd) / 2 + 32 * h + kp] = lo | (hi << 16);
    }
  }
  __syncthreads();
  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < kDownMaxChunk / 32; ++kk) {
    if (kk < nk) {
      const u32x4 fb = *reinterpret_cast<const u32x4*>(&Bt[(wave * 16 + r) * kDownLd + 32 * kk + 8 * g]);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mfma16(fa[t][kk], fb, acc[t]);
    }
  }
  const int col = c0 + wave * 16 + r;
  if (col < d) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * t + 4 * g + e;
        if (tok < B) partial[((int64_t)blockIdx.y * B + tok) * d + col] = acc[t][e];
      }
  }
}

}  // namespace pop
