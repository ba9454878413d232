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
// l & 15.  A fragment load straight from memory would read only 64 contiguous
// bytes of each of 16 rows, so both stages stage the weights through LDS:
// the gate/up rows by LDS-direct loads of whole 128-byte lines, the W_downT
// rows through registers (transposed on the way into LDS).
#pragma once
#include <hip/hip_runtime.h>

#include "partition.h"
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

// Mixture-of-experts form of a launch (kMoe): grid row blockIdx.y is expert e,
// whose weight matrices sit w_stride elements after expert e - 1's, whose
// lists (R, C, and S, positions, scores) are its slices of E stacked lists,
// and whose tokens are the routed pairs offsets[e] .. offsets[e + 1] (pair p
// is token tokens[p]; z row p).  Every expert gets at most as many pairs as
// there are tokens, so the launch's token tiles cover it.
struct MoeRows {
  const int32_t* offsets;
  const int32_t* tokens;
  int64_t w_stride;
};

// Hand-over of the candidate cut inside one launch of k_down_stream (PHASE
// 2): the top-k workgroup publishes it to n_copies words thr[c * stride]
// (coherent), each workgroup polls one copy at most poll_limit times and, if
// that runs out, sets *err to 3 and adds no selected row.
struct CutLink {
  uint64_t* thr;
  uint32_t* err;
  int n_copies, stride, poll_limit;
};

// ---------------------------------------------------------------- gate / up, rows streamed through LDS
// The same product with the weight rows read by LDS-direct loads: one load
// instruction moves 1 KB of one or a few rows (full 128-byte lines; a
// register-fragment load can only cover 64 bytes of each of 16 rows) into a
// ring of kGlNS LDS stages of kGlKC reduction elements, so that many stages
// are in flight without holding registers.
//
// Block b takes the rows [b n_A / nb, (b + 1) n_A / nb) of R u C (at most
// kGlRows; nb is chosen so that every block of the grid is resident at once
// and the rows are balanced).  Wave w computes the 32-wide k-blocks
// w (kGlKC / 128) + [0, kGlKC / 128) of each stage for both row tiles and
// every token tile; the four partial products meet in LDS at the end.
//
// LDS stage layout: [matrix][row][kGlKC] bf16.  Row rho's 16-byte chunk c of
// the stage sits in slot c ^ (rho & 15) (c, slot < kGlKC / 8), so the sixteen
// lanes of a fragment read (rows 16 t + [0, 16), one chunk) hit distinct
// banks.  The load lanes pick their source chunk accordingly: lane slot s of
// row rho loads chunk s ^ (rho & 15).
#ifndef POP_GL_KC
#define POP_GL_KC 256
#endif
#ifndef POP_GL_NS
#define POP_GL_NS 2
#endif
#ifndef POP_GL_ROWS
#define POP_GL_ROWS 24
#endif
#ifndef POP_GL_BLOCKS
#define POP_GL_BLOCKS 512
#endif
constexpr int kGlRows = POP_GL_ROWS;                 // rows per block at most (16 or 24)
constexpr int kGlKC = POP_GL_KC;                     // reduction elements per stage (128 or 256)
constexpr int kGlNS = POP_GL_NS;                     // stages in the LDS ring
constexpr int kGlSlots = kGlKC / 8;                  // 16-byte chunks per row and stage
constexpr int kGlRowsPerLoad = 64 / kGlSlots;        // rows one load instruction covers
constexpr int kGlLoads = 2 * kGlRows / kGlRowsPerLoad / 4;  // load instructions per wave and stage
constexpr int kGlStage = 2 * kGlRows * kGlKC;        // bf16 elements per stage
constexpr int kGlKB = kGlKC / 128;                   // 32-wide k-blocks per wave and stage
static_assert(kGlKC == 128 || kGlKC == 256, "stage width");
static_assert((2 * kGlRows / kGlRowsPerLoad) % 4 == 0, "loads split evenly over the waves");
static_assert(kGlNS >= 2 && kGlNS <= 4, "ring depth");

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt and lgkmcnt at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The host's grid for k_gateup_lds: every block resident (two per CU) and at
// most kGlRows rows each.
__host__ __device__ constexpr int gateup_lds_blocks(int n_A) {
  return (n_A + kGlRows - 1) / kGlRows > POP_GL_BLOCKS ? (n_A + kGlRows - 1) / kGlRows : POP_GL_BLOCKS;
}

template <int MT, bool kIdentity, bool kMoe = false>
__global__ __launch_bounds__(256) void k_gateup_lds(const bf16s* __restrict__ x, int B, int d,
                                                    const bf16s* __restrict__ Wg, const bf16s* __restrict__ Wu,
                                                    int d_ff, const int32_t* __restrict__ R, int n_R,
                                                    const int32_t* __restrict__ C, int n_C, float* __restrict__ z,
                                                    float* __restrict__ score, int nb, MoeRows moe = {}) {
  constexpr int NT = (kGlRows + 15) / 16;  // row tiles
  __shared__ __align__(16) uint16_t smem[kGlNS * kGlStage];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int n_A = n_R + n_C;
  int o0 = 0;  // first routed pair of the expert
  if constexpr (kMoe) {
    const int e = blockIdx.y;
    o0 = moe.offsets[e];
    B = moe.offsets[e + 1] - o0;
    if (B <= 0) return;  // block-uniform: no token reached the expert
    Wg += e * moe.w_stride;
    Wu += e * moe.w_stride;
    R += (int64_t)e * n_R;
    C += (int64_t)e * n_C;
    if (score != nullptr) score += (int64_t)e * n_C;
    z += (int64_t)o0 * n_A;
  }
  const int r0 = (int)((int64_t)blockIdx.x * n_A / nb);
  const int nr = (int)((int64_t)(blockIdx.x + 1) * n_A / nb) - r0;
  if (nr <= 0) return;  // block-uniform
  // load instruction m of this wave: j = wave + 4 m covers matrix j / jm,
  // rows kGlRowsPerLoad (j % jm) + [0, kGlRowsPerLoad) (past nr: the last row)
  constexpr int jm = kGlRows / kGlRowsPerLoad;
  const bf16s* src[kGlLoads];  // the row
  int co[kGlLoads];             // this lane's chunk offset in the stage
  int lds_row[kGlLoads];
  const int slot = lane % kGlSlots;
#pragma unroll
  for (int m = 0; m < kGlLoads; ++m) {
    const int j = wave + 4 * m;
    const int rho = kGlRowsPerLoad * (j % jm) + lane / kGlSlots;
    const int p = r0 + min(rho, nr - 1);
    const int ch = kIdentity ? p : clamp_ch(p < n_R ? R[p] : C[p - n_R], d_ff);
    src[m] = (j < jm ? Wg : Wu) + (int64_t)ch * d;
    co[m] = 8 * (slot ^ (rho & 15));
    lds_row[m] = (j / jm) * kGlRows + kGlRowsPerLoad * (j % jm);  // first row of the instruction
  }
  // this lane's token rows (tokens past B read token 0: never stored)
  const bf16s* xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tok = 16 * t + r < B ? 16 * t + r : 0;
    xr[t] = x + (int64_t)(kMoe ? moe.tokens[o0 + tok] : tok) * d;
  }
  const int nst = (d + kGlKC - 1) / kGlKC;
  u32x4 xs[kGlNS][kGlKB][MT];
  // stage st into ring slot q: this wave's token fragments, then its share of the rows
  auto issue = [&](int st, u32x4 (&xq)[kGlKB][MT], int q) {
    const int kbase = st * kGlKC;
#pragma unroll
    for (int i = 0; i < kGlKB; ++i) {
      const int k = min(kbase + 32 * (kGlKB * wave + i) + 8 * g, d - 8);
#pragma unroll
      for (int t = 0; t < MT; ++t) xq[i][t] = ld16(xr[t] + k);
    }
#pragma unroll
    for (int m = 0; m < kGlLoads; ++m) {
      // chunks past the row's end re-read its last one (their token operands are zero)
      const bf16s* a = src[m] + min(kbase + co[m], d - 8);
      __builtin_amdgcn_global_load_lds((const void*)a,
                                       (__attribute__((address_space(3))) void*)(smem + q * kGlStage +
                                                                                 lds_row[m] * kGlKC),
                                       16, 0, 0);
    }
  };
  f32x4_t ag[NT][MT], au[NT][MT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int t = 0; t < MT; ++t) ag[n][t] = au[n][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto compute = [&](int st, const u32x4 (&xq)[kGlKB][MT], int q) {
    const uint16_t* base = smem + q * kGlStage;
#pragma unroll
    for (int i = 0; i < kGlKB; ++i) {
      const int kb = kGlKB * wave + i;
      const bool on = st * kGlKC + 32 * kb + 8 * g < d;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int row = min(16 * n + r, kGlRows - 1);
        const int sl = (4 * kb + g) ^ (row & 15);
        const u32x4 bg = *reinterpret_cast<const u32x4*>(base + row * kGlKC + 8 * sl);
        const u32x4 bu = *reinterpret_cast<const u32x4*>(base + (kGlRows + row) * kGlKC + 8 * sl);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const u32x4 a = on ? xq[i][t] : zero;
          ag[n][t] = mfma16(a, bg, ag[n][t]);
          au[n][t] = mfma16(a, bu, au[n][t]);
        }
      }
    }
  };
  // Ring: stages 0 .. kGlNS - 2 ahead; step st waits for its own loads (the
  // loads of the later stages already issued may stay in flight), passes a
  // barrier (every wave's share landed, every wave done with stage st - 1),
  // refills stage st - 1's slot with stage st + kGlNS - 1, then computes.
  // The stage count is padded to a multiple of kGlNS (stages past the row's
  // end load its last chunk and compute with zero token operands) and the
  // body is straight-line: the compiler then counts the memory instructions
  // in flight exactly and waits for each token fragment no longer than it
  // must.
  constexpr int kPer = kGlKB * MT + kGlLoads;  // vector-memory instructions per stage
  const int T = (nst + kGlNS - 1) / kGlNS * kGlNS;
  auto step = [&](int st, auto jc, auto issuec, auto laterc) {
    constexpr int j = decltype(jc)::value;
    wait_vmcnt<decltype(laterc)::value * kPer>();
    // the empty asm statements keep every LDS access on its side of the barrier
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(issuec)::value) issue(st + kGlNS - 1, xs[(j + kGlNS - 1) % kGlNS], (j + kGlNS - 1) % kGlNS);
    __builtin_amdgcn_sched_barrier(0);
    compute(st, xs[j], j);
  };
  using std::integral_constant;
#pragma unroll
  for (int j = 0; j < kGlNS - 1; ++j) issue(j, xs[j], j);
  for (int s0 = 0; s0 < T - kGlNS; s0 += kGlNS) {
    step(s0, integral_constant<int, 0>(), integral_constant<bool, true>(), integral_constant<int, kGlNS - 2>());
    step(s0 + 1, integral_constant<int, 1>(), integral_constant<bool, true>(), integral_constant<int, kGlNS - 2>());
    if constexpr (kGlNS > 2)
      step(s0 + 2, integral_constant<int, 2>(), integral_constant<bool, true>(), integral_constant<int, kGlNS - 2>());
    if constexpr (kGlNS > 3)
      step(s0 + 3, integral_constant<int, 3>(), integral_constant<bool, true>(), integral_constant<int, kGlNS - 2>());
  }
  {  // the last group issues only its first step's refill
    const int s0 = T - kGlNS;
    step(s0, integral_constant<int, 0>(), integral_constant<bool, true>(), integral_constant<int, kGlNS - 2>());
    step(s0 + 1, integral_constant<int, 1>(), integral_constant<bool, false>(), integral_constant<int, kGlNS - 2>());
    if constexpr (kGlNS > 2)
      step(s0 + 2, integral_constant<int, 2>(), integral_constant<bool, false>(), integral_constant<int, kGlNS - 3>());
    if constexpr (kGlNS > 3)
      step(s0 + 3, integral_constant<int, 3>(), integral_constant<bool, false>(), integral_constant<int, 0>());
  }
  // the four waves' partial products meet in the (now idle) stage buffers
  wait_vmcnt<0>();
  __syncthreads();
  f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);  // [wave - 1][2 NT MT][64]
  static_assert(3 * 2 * NT * 4 * 64 * 16 <= kGlNS * kGlStage * 2, "reduction fits the ring");
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        red[((wave - 1) * 2 * NT * MT + 2 * (n * MT + t)) * 64 + lane] = ag[n][t];
        red[((wave - 1) * 2 * NT * MT + 2 * (n * MT + t) + 1) * 64 + lane] = au[n][t];
      }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float smax = 0.f;
    const int rl = 16 * n + r;
    const int prow = r0 + rl;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      f32x4_t gs = ag[n][t], us = au[n][t];
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        gs += red[(w * 2 * NT * MT + 2 * (n * MT + t)) * 64 + lane];
        us += red[(w * 2 * NT * MT + 2 * (n * MT + t) + 1) * 64 + lane];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * t + 4 * g + e;
        if (tok < B) {
          const float zz = silu(gs[e]) * us[e];
          if (rl < nr) z[(int64_t)tok * n_A + prow] = zz;
          smax = fmaxf(smax, fabsf(zz));
        }
      }
    }
    smax = fmaxf(smax, __shfl_xor(smax, 16));
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    if (g == 0 && rl < nr && prow >= n_R && score != nullptr) score[prow - n_R] = smax;
  }
}

// ---------------------------------------------------------------- down, streamed
// Block (slice, chunk): output columns slice * 64 + [0, 64) over the live
// rows q0 = row_begin + chunk * rows_per_chunk + [0, rows_per_chunk)
// (clipped at row_end; at most kDsMaxRows), taken as sub-chunks of kDsRows
// rows in a pipelined loop that keeps the products of all sub-chunks in the
// accumulators: one partial sum per block, however long its range.
//   * The range's channels and z columns go to LDS first (one round trip);
//     live row q is (R[q], q) for q < n_R and (sel[q - n_R], n_R + pos[q - n_R])
//     after, or (q, q) with kIdentity.
//   * A ring of kDsNS sub-chunks of loads is in flight in registers: each
//     thread's two rows (pairs 2 (t >> 3) + [0, 2), eight lanes per row read
//     its 128 contiguous bytes of the slice) and the z values of its row pair
//     for its tokens.
//   * Each sub-chunk goes to LDS (double-buffered, one barrier per
//     sub-chunk): rows transposed as (row, row + 1) pairs into Bt[column][row]
//     with the pair index XOR-swizzled by 4 ((column >> 3) & 7) (conflict-free
//     writes), z rounded to bf16 into zs[token][row]; then the four waves run
//     their 16 columns' products.
// Rows past the range read its last row with z = 0; columns past d and tokens
// past B read valid memory and produce outputs that are never stored.
//
// PHASE 1: blocks [0, nb0) run the candidate top-k instead (one block), so it
// overlaps the retained rows' product; the selected rows follow in a PHASE 0
// launch.
// PHASE 2: as PHASE 1, but the top-k block publishes the cut (CutLink) before
// it writes the lists;
// after its retained rows, block (slice, chunk) takes the chunk's even share
// of the candidate positions (n_A - n_R of them), keeps those the cut selects
// (in position order) and streams their W_downT rows into the same
// accumulators: one launch and one partial per block for R and S together.
// PHASE 3: the same rows from a given selection (sel and pos, positions
// ascending) instead of a top-k: the same sums, bit for bit.
#ifndef POP_DS_NS
#define POP_DS_NS 4
#endif
constexpr int kDsRows = 64;                // rows per sub-chunk
constexpr int kDsMaxRows = 1024;           // rows per block at most
constexpr int kDsNS = POP_DS_NS;           // sub-chunks of loads in flight
constexpr int kDsLd = kDsRows + 8;         // Bt and zs pitch in bf16 (144 bytes)
static_assert(kDsNS >= 2 && kDsNS <= 4, "ring depth");

template <int MT>
struct DsShared {
  uint16_t Bt[2][64 * kDsLd];       // [column][row of the sub-chunk]
  uint16_t zs[2][16 * MT * kDsLd];  // [token][row of the sub-chunk]
  int rch[kDsMaxRows];
  int zcol[kDsMaxRows];
  uint64_t cut;  // PHASE 2: the cut as read
  int wsum[4];   // PHASE 2: selected candidates per wave
};

template <int MT, bool kIdentity, int PHASE, bool kMoe = false>
__global__ __launch_bounds__(256) void k_down_stream(const float* __restrict__ z, int n_A, int B,
                                                     const bf16s* __restrict__ WdT, int d, int d_ff,
                                                     const int32_t* __restrict__ R, int n_R,
                                                     const int32_t* __restrict__ sel, const int32_t* __restrict__ pos,
                                                     int row_begin, int row_end, int rows_per_chunk, int chunk_base,
                                                     float* __restrict__ partial, int nb0,
                                                     const float* __restrict__ score, int n_C, int k,
                                                     const int32_t* __restrict__ C, int32_t* __restrict__ Q,
                                                     int32_t* __restrict__ S, CutLink link, MoeRows moe = {}) {
  using DS = DsShared<MT>;
  // the top-k block (up to 4096 candidates)
  constexpr size_t kTs = PHASE == 1 ? topk_lds_bytes<256>(4096) : PHASE == 2 ? sizeof(SelShared<256, 4096>) : 0;
  constexpr size_t kSmem = sizeof(DS) > kTs ? sizeof(DS) : kTs;
  __shared__ __align__(16) unsigned char smem[kSmem];
  int o0 = 0, cnt = B;  // the launch's z rows: all B, or the expert's routed pairs (B = every pair)
  if constexpr (kMoe) {
    const int e = blockIdx.y;
    o0 = moe.offsets[e];
    cnt = moe.offsets[e + 1] - o0;
    if (cnt <= 0) return;  // block-uniform: no token reached the expert
    WdT += e * moe.w_stride;
    R += (int64_t)e * n_R;
    sel += (int64_t)e * k;
    pos += (int64_t)e * k;
    C += (int64_t)e * n_C;
    Q += (int64_t)e * k;
    S += (int64_t)e * k;
    if (score != nullptr) score += (int64_t)e * n_C;
    z += (int64_t)o0 * n_A;
  }
  if constexpr (PHASE == 1) {
    if ((int)blockIdx.x < nb0) {
      topk_select<256>(score, n_C, k, C, Q, S, smem);
      return;
    }
  }
  if constexpr (PHASE == 2) {
    if ((int)blockIdx.x < nb0) {  // the cut first (published), then the lists
      topk_threshold_linked<256, 4096>(nullptr, n_C, k, C, Q, S, link.thr, link.n_copies, link.stride,
                                       *reinterpret_cast<SelShared<256, 4096>*>(smem), link.poll_limit, link.err,
                                       score);
      return;
    }
  }
  DS& sh = *reinterpret_cast<DS*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int ncol = (d + 63) / 64;
  const int idx = (int)blockIdx.x - (PHASE >= 1 ? nb0 : 0);
  const int c0 = (idx % ncol) * 64;
  const int cl = idx / ncol;
  const int q0 = row_begin + cl * rows_per_chunk;
  int nrows = min(row_end, q0 + rows_per_chunk) - q0;  // >= 1: the host launches no empty chunk
  // PHASE >= 2: this chunk's share [ca, cb) of the candidate positions; PHASE
  // 2 reads their scores now, long before it needs them
  const int nchunks = (row_end - row_begin + rows_per_chunk - 1) / rows_per_chunk;
  const int ca = (int)((int64_t)(n_A - n_R) * cl / nchunks), cb = (int)((int64_t)(n_A - n_R) * (cl + 1) / nchunks);
  constexpr int kScPer = kDsMaxRows / 256;
  uint32_t scv[kScPer];
#pragma unroll
  for (int u = 0; u < kScPer; ++u) scv[u] = 0u;
  if constexpr (PHASE == 2) {
#pragma unroll
    for (int u = 0; u < kScPer; ++u) scv[u] = value_bits(score[min(ca + kScPer * tid + u, max(cb - 1, 0))]);
  }
  {  // every index load in flight at once (clamped to the range; stores masked)
    constexpr int kPer = kDsMaxRows / 256;
    int a[kPer], b[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int q = q0 + min(tid + 256 * u, nrows - 1);
      if (kIdentity) {
        a[u] = q;
        b[u] = q;
      } else if (q < n_R) {  // a chunk holds retained or selected rows only
        a[u] = R[q];
        b[u] = q;
      } else {
        a[u] = sel[q - n_R];
        b[u] = pos[q - n_R];
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + 256 * u;
      if (i < nrows) {
        sh.rch[i] = kIdentity ? a[u] : clamp_ch(a[u], d_ff);
        sh.zcol[i] = (kIdentity || q0 < n_R) ? b[u] : min(n_R + max(b[u], 0), n_A - 1);
      }
    }
  }
  __syncthreads();
  // loads: row pair kp (rows 2 kp, 2 kp + 1 of a sub-chunk), columns cc + [0, 8)
  const int kp = tid >> 3, cc = (tid & 7) * 8;
  const bf16s* wcol = WdT + min(c0 + cc, d - 8);
  // z: row pair zp (rows 2 zp, 2 zp + 1), tokens zt + 8 m
  const int zp = tid & 31, zt = tid >> 5;
  struct Ld {
    u32x4 va, vb;
    float za[2 * MT], zb[2 * MT];
  };
  auto issue = [&](int i, Ld& L) {
    const int ra = min(kDsRows * i + 2 * kp, nrows - 1), rb = min(kDsRows * i + 2 * kp + 1, nrows - 1);
    L.va = ld16(wcol + (int64_t)sh.rch[ra] * d);
    L.vb = ld16(wcol + (int64_t)sh.rch[rb] * d);
    const int ca = sh.zcol[min(kDsRows * i + 2 * zp, nrows - 1)];
    const int cb = sh.zcol[min(kDsRows * i + 2 * zp + 1, nrows - 1)];
#pragma unroll
    for (int m = 0; m < 2 * MT; ++m) {
      const float* zr = z + (int64_t)min(zt + 8 * m, cnt - 1) * n_A;
      L.za[m] = zr[ca];
      L.zb[m] = zr[cb];
    }
  };
  auto put = [&](int i, const Ld& L, int buf) {
    uint32_t* b32 = reinterpret_cast<uint32_t*>(sh.Bt[buf]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = cc + j;
      const uint32_t lo = (L.va[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
      const uint32_t hi = (L.vb[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
      b32[col * (kDsLd / 2) + (kp ^ (4 * ((col >> 3) & 7)))] = lo | (hi << 16);
    }
    const bool on0 = kDsRows * i + 2 * zp < nrows, on1 = kDsRows * i + 2 * zp + 1 < nrows;
    uint32_t* z32 = reinterpret_cast<uint32_t*>(sh.zs[buf]);
#pragma unroll
    for (int m = 0; m < 2 * MT; ++m)
      z32[(zt + 8 * m) * (kDsLd / 2) + zp] = bf16_pack_rne(on0 ? L.za[m] : 0.f, on1 ? L.zb[m] : 0.f);
  };
  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int bcol = wave * 16 + r;
  const int bsw = 4 * ((bcol >> 3) & 7);
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kDsRows / 32; ++kk) {
      const uint32_t* b32 = reinterpret_cast<const uint32_t*>(sh.Bt[buf]);
      const u32x4 fb = *reinterpret_cast<const u32x4*>(b32 + bcol * (kDsLd / 2) + ((16 * kk + 4 * g) ^ bsw));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const u32x4 fa = *reinterpret_cast<const u32x4*>(&sh.zs[buf][(16 * t + r) * kDsLd + 32 * kk + 8 * g]);
        acc[t] = mfma16(fa, fb, acc[t]);
      }
    }
  };
  // Straight-line ring (the count of sub-chunks padded to a multiple of the
  // ring depth; padded ones carry z = 0): the compiler then waits for each
  // sub-chunk's loads and no more.
  Ld ring[kDsNS];
  uint64_t cw = 0;  // PHASE 2: the cut as last read, beside every step's loads
  const uint64_t* cutp = PHASE == 2 ? link.thr + (int64_t)(idx % max(link.n_copies, 1)) * link.stride : nullptr;
  static_assert(kDsNS % 2 == 0, "the LDS buffer of step i is i & 1 = j & 1");
  using std::integral_constant;
  // One pass over the rows in sh.rch / sh.zcol [0, nrows) with a ring of NS
  // sub-chunks (NS even, at most kDsNS).
  auto ring_pass = [&](auto nsc) {
    constexpr int NS = decltype(nsc)::value;
    static_assert(NS % 2 == 0 && NS <= kDsNS, "ring depth");
    auto step = [&](int i, auto jc, auto issuec) {
      constexpr int j = decltype(jc)::value;
      // the scheduling barriers keep each step's unpacking after the loads it
      // waits for were given their time (no hoisting of a later step's work)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(issuec)::value) issue(i + NS - 1, ring[(j + NS - 1) % NS]);
      if constexpr (PHASE == 2) cw = ld_coh(cutp);
      __builtin_amdgcn_sched_barrier(0);
      put(i, ring[j], j & 1);
      // LDS only: the later sub-chunks' loads stay in flight across it (a
      // workgroup-release barrier would wait for all of them at every step).
      // The buffer put(i + 1) writes was last read by compute(i - 1), which
      // every wave finished before this barrier of step i.
      lds_barrier();
      compute(j & 1);
    };
    const int nsub = (nrows + kDsRows - 1) / kDsRows;
    const int T = (nsub + NS - 1) / NS * NS;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(j, ring[j]);
    for (int i0 = 0; i0 < T - NS; i0 += NS) {
      step(i0, integral_constant<int, 0>(), integral_constant<bool, true>());
      step(i0 + 1, integral_constant<int, 1>(), integral_constant<bool, true>());
      if constexpr (NS > 2) {
        step(i0 + 2, integral_constant<int, 2>(), integral_constant<bool, true>());
        step(i0 + 3, integral_constant<int, 3>(), integral_constant<bool, true>());
      }
    }
    {
      const int i0 = T - NS;
      step(i0, integral_constant<int, 0>(), integral_constant<bool, true>());
      step(i0 + 1, integral_constant<int, 1>(), integral_constant<bool, false>());
      if constexpr (NS > 2) {
        step(i0 + 2, integral_constant<int, 2>(), integral_constant<bool, false>());
        step(i0 + 3, integral_constant<int, 3>(), integral_constant<bool, false>());
      }
    }
  };
  ring_pass(integral_constant<int, kDsNS>());
  if constexpr (PHASE >= 2) {
    // then the chunk's selected candidates: those at positions in the
    // chunk's share [ca, cb) of C, in position order, as one more pass (the
    // host keeps every share within kDsMaxRows candidates)
    int ns = 0;
    if constexpr (PHASE == 2) {  // from the scores and the cut, handed over inside this launch
      // thread 0's last read decides for the workgroup (the waves read the
      // cut at different times); poll only if it was not out yet
      if (tid == 0) {
        bool ok = true;
        const uint64_t e = is_valid(cw) ? cw : poll_coh(cutp, [](uint64_t v) { return is_valid(v); },
                                                         link.poll_limit, ok);
        if (!ok) st_coh(link.err, 3u);
        sh.cut = ok ? e : 0;
      }
      __syncthreads();  // also: every wave is past the first pass's reads of the lists
      const uint64_t e = sh.cut;
      const uint32_t cv = (uint32_t)(e >> 32) & 0x7fffffffu;
      const int tie = (int)(uint32_t)e;
      int fl = 0, cnt = 0;
#pragma unroll
      for (int u = 0; u < kScPer; ++u) {
        const int i = ca + kScPer * tid + u;
        if (is_valid(e) && i < cb && (scv[u] > cv || (scv[u] == cv && i <= tie))) {
          fl |= 1 << u;
          ++cnt;
        }
      }
      const int incl = wave_incl_scan(cnt);
      if (lane == 63) sh.wsum[wave] = incl;
      __syncthreads();
      int off = incl - cnt;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        off += w < wave ? sh.wsum[w] : 0;
        ns += sh.wsum[w];
      }
#pragma unroll
      for (int u = 0; u < kScPer; ++u)
        if ((fl >> u) & 1) {
          const int i = ca + kScPer * tid + u;
          sh.rch[off] = clamp_ch(C[i], d_ff);
          sh.zcol[off] = min(n_R + i, n_A - 1);
          ++off;
        }
    } else {  // from the selected list (positions ascending): the entries [ja, jb) fall in the share
      if (tid < 2) sh.wsum[tid] = 0;
      __syncthreads();  // also: every wave is past the first pass's reads of the lists
      int lo = 0, hi = 0;
      for (int j = tid; j < k; j += 256) {
        const int p = pos[j];
        lo += p < ca ? 1 : 0;
        hi += p < cb ? 1 : 0;
      }
      if (lo) atomicAdd(&sh.wsum[0], lo);
      if (hi) atomicAdd(&sh.wsum[1], hi);
      __syncthreads();
      const int ja = sh.wsum[0];
      ns = min(sh.wsum[1] - ja, kDsMaxRows);
      for (int i = tid; i < ns; i += 256) {
        sh.rch[i] = clamp_ch(sel[ja + i], d_ff);
        sh.zcol[i] = min(n_R + max(pos[ja + i], 0), n_A - 1);
      }
    }
    __syncthreads();
    if (ns > 0) {  // block-uniform: a shallow ring for these few sub-chunks
      nrows = ns;
      ring_pass(integral_constant<int, 2>());
    }
  }
  const int col = c0 + bcol;
  if (col < d) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * t + 4 * g + e;
        if (tok < cnt) partial[((int64_t)(chunk_base + cl) * B + o0 + tok) * d + col] = acc[t][e];
      }
  }
}

}  // namespace pop
