// Dense gated MLP over the prompt tokens: the prefill forward that precedes
// the pruned decode (POP notes, "Loss / training strategy": the online masking
// starts from the second step, so the prompt's own FFN runs dense).  The gated
// MLP is equation (1) of "Batch-wise adaptive pruning ... for language
// reasoning models", section 3.1:
//
//   Z = SiLU(X W_gate^T) * (X W_up^T)      [n_tokens, d_ff]   (workspace)
//   Y = Z W_down^T = Z W_downT             [n_tokens, d]      fp32
//
// bf16: two MFMA GEMMs (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Z is
// stored in bf16 (round to nearest even), the operand type of the second GEMM.
// fp32: the same two products as LDS-tiled fp32 FMA.
//
// Both bf16 GEMMs use 256-thread blocks of 128 tokens x 64 output columns and a
// 64-wide reduction slice per stage: each stage's global loads go to a ring of
// register slots (2 for gate/up, 4 for the down-projection) and stay in flight
// under the MFMAs of the stages before it; a stage then moves to one of two
// LDS buffers.  Whole stages load with no condition (clamped rows and
// channels), which keeps the compiler from waiting on the loads in flight.
// Every operand tile is stored K-contiguous in LDS with a 144-byte row pitch,
// which makes the 16-lane groups of a fragment read hit all 64 banks once.
// W_downT is [d_ff, d] (K-major for the second GEMM), so its tile is
// transposed on the way into LDS.
#include <hip/hip_runtime.h>

#include "pop_device.h"
#include "pop_internal.h"
#include "prompt_gemm.h"

namespace pop {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGThreads = 256;
constexpr int kBM = 128;         // tokens per block
constexpr int kBN = 64;          // output columns per block (per matrix)
constexpr int kBK = 64;          // reduction slice per stage
constexpr int kLd = kBK + 8;     // LDS row pitch in bf16 elements (144 bytes)
constexpr int kZPad = 64;        // Z row pitch = d_ff rounded up to this
constexpr int64_t kChunkTokens = 4096;  // tokens per pass (bounds the workspace)
#ifndef POP_GATEUP_NS
#define POP_GATEUP_NS 2  // register stages of the gate/up pass's load pipeline (3 drops to one wave per SIMD)
#endif
#ifndef POP_DOWN_NS
#define POP_DOWN_NS 4  // register stages of the down-projection's load pipeline
#endif
#ifndef POP_DOWN_BM64_BELOW
#define POP_DOWN_BM64_BELOW 0  // down-projection tiles of 128 tokens below which 64-token tiles are used
#endif

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Tile order: workgroups are handed to the eight XCDs round robin by index, so
// block b runs on XCD b % 8.  Tiles are renumbered so that each XCD takes a
// contiguous run of tiles in (token tile fastest) order: the token tiles that
// share one weight tile run on the same XCD, close in time, and share its L2.
__device__ __forceinline__ void tile_of(int bid, int nb, int mt, int& m_tile, int& n_tile) {
  const int nb8 = nb & ~7;
  const int q = bid < nb8 ? (bid & 7) * (nb8 >> 3) + (bid >> 3) : bid;
  m_tile = q % mt;
  n_tile = q / mt;
}

// ---------------------------------------------------------------- gate / up
// Wave w covers tokens (w >> 1) * 64 + [0, 64) and channels (w & 1) * 32 +
// [0, 32) of the block's tile, for both matrices: 4 x 2 fragments each.
//
// IMP > 0: the blocks also compute the importance
// I_i = sqrt(sum_k W_up[i,k]^2 * s2[k]) of the block's channels from the W_up
// tiles already in LDS (the column norms s2 of the whole prompt are an input),
// so the prefill needs no second sweep of W_up.  IMP = 16: the blocks of the
// first four token tiles take 16 of the 64 channels each (m_tile * 16 + [0,
// 16)), so the extra work is spread evenly; IMP = 64 (fewer than four token
// tiles): the first token tile takes all 64.  Thread t takes channel
// t % IMP and the KPT = 64 * IMP / 256 columns (t / IMP) * KPT + [0, KPT) of
// every 64-column stage, in ascending order; the 256 / IMP column groups of a
// channel are added in order at the end.
//
// Pipeline (as in the down-projection): each stage's loads go to one of NS
// register slots and stay in flight for NS - 1 stages of MFMA work, then the
// stage is written to one of two LDS buffers, followed by one barrier.  The
// stages that lie wholly below d (in groups of NS) load unconditionally: rows
// past M are clamped to row M - 1 (their outputs are not written) and channels
// past d_ff to channel d_ff - 1 (their Z columns are written as 0 below).  The
// last stages (fewer than NS, or a stage that crosses d) load with a column
// mask so that columns past d are 0, one stage at a time.
template <int IMP, int NS>
__global__ __launch_bounds__(kGThreads) void k_prompt_gateup(const bf16s* __restrict__ X, int M, int d,
                                                             const bf16s* __restrict__ Wg,
                                                             const bf16s* __restrict__ Wu, int d_ff,
                                                             uint16_t* __restrict__ Z, int ldz, int mt, int nt,
                                                             const float* __restrict__ s2, float* __restrict__ I) {
  __shared__ __align__(16) uint16_t As[2][kBM * kLd];
  __shared__ __align__(16) uint16_t Bs[2][2 * kBN * kLd];  // gate rows, then up rows
  constexpr int APER = kBM * (kBK / 8) / kGThreads;
  constexpr int BPER = 2 * kBN * (kBK / 8) / kGThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int m_tile, n_tile;
  tile_of(blockIdx.x, mt * nt, mt, m_tile, n_tile);
  const int m0 = m_tile * kBM, n0 = n_tile * kBN;
  const int wm = wave >> 1, wn = wave & 1;

  // importance state (block-uniform)
  constexpr int IC = IMP > 0 ? IMP : 64;       // channels per importance block
  constexpr int KPT = 64 * IC / kGThreads;     // columns per thread per stage (4 or 16)
  constexpr int SPS = IMP > 0 ? KPT : 1;       // s2 values per slot
  const bool imp = IMP > 0 && m_tile < (IMP == 16 ? 4 : 1);
  const int c_base = IMP == 16 ? m_tile * 16 : 0;
  const int ir = tid % IC, ig = tid / IC;
  float ia = 0.f;

  u32x4 ra[NS][APER], rb[NS][BPER];
  float rs[NS][SPS];
  // Whole stages: unconditional loads.  Columns of s2 past d are read at
  // d - 4 (finite); they only ever meet W_up columns that are 0 in LDS.
  auto issue = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int q = tid + i * kGThreads;
      const int m = min(m0 + (q >> 3), M - 1);
      ra[slot][i] = ld16(X + (int64_t)m * d + k0 + (q & 7) * 8);
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int q = tid + i * kGThreads;
      const int row = q >> 3;
      const int ch = min(n0 + (row & (kBN - 1)), d_ff - 1);
      const bf16s* W = row < kBN ? Wg : Wu;
      rb[slot][i] = ld16(W + (int64_t)ch * d + k0 + (q & 7) * 8);
    }
    if constexpr (IMP > 0) {
#pragma unroll
      for (int q = 0; q < KPT; q += 4) {
        const float4 f = *reinterpret_cast<const float4*>(s2 + min(k0 + ig * KPT + q, d - 4));
        rs[slot][q] = f.x;
        rs[slot][q + 1] = f.y;
        rs[slot][q + 2] = f.z;
        rs[slot][q + 3] = f.w;
      }
    }
  };
  // Tail stages: columns past d load as 0.
  auto issue_masked = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int q = tid + i * kGThreads;
      const int m = min(m0 + (q >> 3), M - 1), k = k0 + (q & 7) * 8;
      ra[slot][i] = k < d ? ld16(X + (int64_t)m * d + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int q = tid + i * kGThreads;
      const int row = q >> 3, k = k0 + (q & 7) * 8;
      const int ch = min(n0 + (row & (kBN - 1)), d_ff - 1);
      const bf16s* W = row < kBN ? Wg : Wu;
      rb[slot][i] = k < d ? ld16(W + (int64_t)ch * d + k) : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (IMP > 0) {
#pragma unroll
      for (int q = 0; q < KPT; q += 4) {
        const float4 f = *reinterpret_cast<const float4*>(s2 + min(k0 + ig * KPT + q, d - 4));
        rs[slot][q] = f.x;
        rs[slot][q + 1] = f.y;
        rs[slot][q + 2] = f.z;
        rs[slot][q + 3] = f.w;
      }
    }
  };
  auto put = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int q = tid + i * kGThreads;
      *reinterpret_cast<u32x4*>(&As[buf][(q >> 3) * kLd + (q & 7) * 8]) = ra[slot][i];
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int q = tid + i * kGThreads;
      *reinterpret_cast<u32x4*>(&Bs[buf][(q >> 3) * kLd + (q & 7) * 8]) = rb[slot][i];
    }
  };

  f32x4 ag[4][2], au[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ag[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  auto compute = [&](int slot, int buf) {
    if constexpr (IMP > 0) {
      // W_up row n0 + c_base + ir of this stage: columns ig * KPT + [0, KPT)
      const uint16_t* wr = &Bs[buf][(kBN + c_base + ir) * kLd + ig * KPT];
#pragma unroll
      for (int q = 0; q < KPT; q += 2) {
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(wr + q);
        const float f0 = __uint_as_float(w2 << 16), f1 = __uint_as_float(w2 & 0xffff0000u);
        ia = fmaf(f0 * f0, rs[slot][q], ia);
        ia = fmaf(f1 * f1, rs[slot][q + 1], ia);
      }
    }
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds_frag(&As[buf][(wm * 64 + i * 16 + fr) * kLd + kk + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 fg = lds_frag(&Bs[buf][(wn * 32 + j * 16 + fr) * kLd + kk + fk]);
        const bf16x8 fu = lds_frag(&Bs[buf][(kBN + wn * 32 + j * 16 + fr) * kLd + kk + fk]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ag[i][j] = mfma(fa[i], fg, ag[i][j]);
          au[i][j] = mfma(fa[i], fu, au[i][j]);
        }
      }
    }
  };

  const int nk = (d + kBK - 1) / kBK;
  const int nmain = d / kBK / NS * NS;  // whole stages, in groups of NS
  if (nmain > 0) {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) issue(u, u * kBK);
  }
  for (int kt0 = 0; kt0 < nmain; kt0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int kt = kt0 + u;
      issue((u + NS - 1) % NS, min(kt + NS - 1, nmain - 1) * kBK);  // past the end: reload (unused)
      put(u, kt & 1);
      __syncthreads();
      compute(u, kt & 1);
    }
  }
  for (int kt = nmain; kt < nk; ++kt) {  // the last stages, one at a time
    issue_masked(0, kt * kBK);
    put(0, kt & 1);
    __syncthreads();
    compute(0, kt & 1);
  }
  __syncthreads();  // every wave is done with As before it holds the importance sums
  if (imp) {  // block-uniform
    float* red = reinterpret_cast<float*>(As[0]);
    red[ig * IC + ir] = ia;
    __syncthreads();
    if (ig == 0 && n0 + c_base + ir < d_ff) {
      float t = red[ir];
#pragma unroll
      for (int g = 1; g < kGThreads / IC; ++g) t += red[g * IC + ir];
      I[n0 + c_base + ir] = sqrtf(t);
    }
  }
  // Output fragment layout: element e of lane l is row (l >> 4) * 4 + e,
  // column l & 15 of the 16 x 16 tile.  Columns in [d_ff, ldz) are written as
  // 0: Z's padding must be zero for the second GEMM.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 32 + j * 16 + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        if (m < M && n < ldz)
          Z[(int64_t)m * ldz + n] = n < d_ff ? bf16_rne(silu(ag[i][j][e]) * au[i][j][e]) : (uint16_t)0;
      }
    }
}

// ---------------------------------------------------------------- down
// Y[m, n] = sum_k Z[m, k] W_downT[k, n].  The W_downT tile (kBK rows of kBN
// columns, row-major in HBM) is written to LDS as [n][k]: thread t loads rows
// k0 + 2 (t & 31) and the next one at columns (t >> 5) * 8 + [0, 8) and writes
// eight 4-byte (k, k + 1) pairs; the 32 k-pairs of a half-wave cover all 64
// banks.  BM = 128: wave w covers tokens (w >> 1) * 64 + [0, 64) and columns
// (w & 1) * 32 + [0, 32); BM = 64 (twice the blocks, for short prompts): wave w
// covers all 64 tokens and columns w * 16 + [0, 16).
//
// Pipeline: the loads of a stage go to one of NS register slots and stay in
// flight for NS - 1 stages of MFMA work (a stage's loads take far longer than
// its arithmetic); each stage is then written to one of two LDS buffers,
// followed by one barrier.  Every load is unconditional: a Z row past M is
// clamped to row M - 1 (it only feeds output rows that are not written),
// W_downT rows past d_ff are clamped to row d_ff - 1 (they meet Z's zero
// padding) and columns past d to the last vector (their outputs are not
// written).  No branch or select follows a load.
template <int BM, int NS>
__global__ __launch_bounds__(kGThreads) void k_prompt_down(const uint16_t* __restrict__ Z, int M, int ldz,
                                                           const bf16s* __restrict__ WdT, int d_ff, int d,
                                                           float* __restrict__ Y, int mt, int nt) {
  constexpr int WM = BM / 64;            // waves along the tokens
  constexpr int WN = 4 / WM;             // waves along the columns
  constexpr int JF = kBN / WN / 16;      // 16-column fragments per wave
  constexpr int PER = BM * (kBK / 8) / kGThreads;
  __shared__ __align__(16) uint16_t As[2][BM * kLd];
  __shared__ __align__(16) uint16_t Bs[2][kBN * kLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int m_tile, n_tile;
  tile_of(blockIdx.x, mt * nt, mt, m_tile, n_tile);
  const int m0 = m_tile * BM, n0 = n_tile * kBN;
  const int wm = wave / WN, wn = wave % WN;
  const int kp = tid & 31, cb = (tid >> 5) * 8;
  const bf16s* Zb = reinterpret_cast<const bf16s*>(Z);
  const int nb = min(n0 + cb, d - 8);

  u32x4 ra[NS][PER], rb0[NS], rb1[NS];
  auto issue = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * kGThreads;
      const int m = min(m0 + (q >> 3), M - 1);
      ra[slot][i] = ld16(Zb + (int64_t)m * ldz + k0 + (q & 7) * 8);
    }
    const int k = min(k0 + 2 * kp, d_ff - 1), k1 = min(k0 + 2 * kp + 1, d_ff - 1);
    rb0[slot] = ld16(WdT + (int64_t)k * d + nb);
    rb1[slot] = ld16(WdT + (int64_t)k1 * d + nb);
  };
  auto put = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * kGThreads;
      *reinterpret_cast<u32x4*>(&As[buf][(q >> 3) * kLd + (q & 7) * 8]) = ra[slot][i];
    }
    uint32_t* s32 = reinterpret_cast<uint32_t*>(Bs[buf]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = (rb0[slot][j >> 1] >> ((j & 1) * 16)) & 0xffffu;
      const uint32_t hi = (rb1[slot][j >> 1] >> ((j & 1) * 16)) & 0xffffu;
      s32[((cb + j) * kLd) / 2 + kp] = lo | (hi << 16);
    }
  };
  f32x4 acc[4][JF];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds_frag(&As[buf][(wm * 64 + i * 16 + fr) * kLd + kk + fk]);
#pragma unroll
      for (int j = 0; j < JF; ++j) {
        const bf16x8 fb = lds_frag(&Bs[buf][(wn * JF * 16 + j * 16 + fr) * kLd + kk + fk]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma(fa[i], fb, acc[i][j]);
      }
    }
  };

  const int nk = (d_ff + kBK - 1) / kBK;  // Z's pitch ldz >= nk * kBK, its padding is zero
  const int nmain = nk / NS * NS;
  if (nmain > 0) {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) issue(u, u * kBK);
  }
  for (int kt0 = 0; kt0 < nmain; kt0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int kt = kt0 + u;
      issue((u + NS - 1) % NS, min(kt + NS - 1, nmain - 1) * kBK);  // past the end: reload (unused)
      put(u, kt & 1);
      __syncthreads();
      compute(kt & 1);
    }
  }
  for (int kt = nmain; kt < nk; ++kt) {  // fewer than NS stages left
    issue(0, kt * kBK);
    put(0, kt & 1);
    __syncthreads();
    compute(kt & 1);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JF; ++j) {
      const int n = n0 + wn * JF * 16 + j * 16 + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        if (m < M && n < d) Y[(int64_t)m * d + n] = acc[i][j][e];
      }
    }
}

// ---------------------------------------------------------------- fp32
// 16 x 16 output tiles, 16-wide reduction slices staged in LDS; thread (ty, tx)
// owns output (m0 + ty, n0 + tx).
constexpr int kFT = 16;

// kImp: the blocks of the first token tile also compute I for their 16
// channels (thread (ty, tx) sums column tx of channel n0 + ty over the
// stages; the 16 partial sums of a channel are added in column order).
template <bool kImp>
__global__ __launch_bounds__(kFT* kFT) void k_prompt_gateup_f32(const float* __restrict__ X, int M, int d,
                                                                 const float* __restrict__ Wg,
                                                                 const float* __restrict__ Wu, int d_ff,
                                                                 float* __restrict__ Z, int ldz,
                                                                 const float* __restrict__ s2,
                                                                 float* __restrict__ I) {
  __shared__ float xs[kFT][kFT + 1], gs[kFT][kFT + 1], us[kFT][kFT + 1];
  const int tx = threadIdx.x % kFT, ty = threadIdx.x / kFT;
  const int m0 = blockIdx.y * kFT, n0 = blockIdx.x * kFT;
  const bool imp = kImp && blockIdx.y == 0;
  float g = 0.f, u = 0.f, ia = 0.f;
  for (int k0 = 0; k0 < d; k0 += kFT) {
    const int k = k0 + tx;
    xs[ty][tx] = (m0 + ty < M && k < d) ? X[(int64_t)(m0 + ty) * d + k] : 0.f;
    gs[ty][tx] = (n0 + ty < d_ff && k < d) ? Wg[(int64_t)(n0 + ty) * d + k] : 0.f;
    us[ty][tx] = (n0 + ty < d_ff && k < d) ? Wu[(int64_t)(n0 + ty) * d + k] : 0.f;
    __syncthreads();
    if (imp) ia = fmaf(us[ty][tx] * us[ty][tx], k < d ? s2[k] : 0.f, ia);
#pragma unroll
    for (int j = 0; j < kFT; ++j) {
      g = fmaf(xs[ty][j], gs[tx][j], g);
      u = fmaf(xs[ty][j], us[tx][j], u);
    }
    __syncthreads();
  }
  const int m = m0 + ty, n = n0 + tx;
  if (m < M && n < d_ff) Z[(int64_t)m * ldz + n] = silu(g) * u;
  if (imp) {  // block-uniform
    xs[ty][tx] = ia;
    __syncthreads();
    if (tx == 0 && n0 + ty < d_ff) {
      float t = xs[ty][0];
#pragma unroll
      for (int j = 1; j < kFT; ++j) t += xs[ty][j];
      I[n0 + ty] = sqrtf(t);
    }
  }
}

__global__ __launch_bounds__(kFT* kFT) void k_prompt_down_f32(const float* __restrict__ Z, int M, int ldz,
                                                              const float* __restrict__ WdT, int d_ff, int d,
                                                              float* __restrict__ Y) {
  __shared__ float zs[kFT][kFT + 1], ws[kFT][kFT + 1];
  const int tx = threadIdx.x % kFT, ty = threadIdx.x / kFT;
  const int m0 = blockIdx.y * kFT, n0 = blockIdx.x * kFT;
  float acc = 0.f;
  for (int k0 = 0; k0 < d_ff; k0 += kFT) {
    zs[ty][tx] = (m0 + ty < M && k0 + tx < d_ff) ? Z[(int64_t)(m0 + ty) * ldz + k0 + tx] : 0.f;
    ws[ty][tx] = (k0 + ty < d_ff && n0 + tx < d) ? WdT[(int64_t)(k0 + ty) * d + n0 + tx] : 0.f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kFT; ++j) acc = fmaf(zs[ty][j], ws[j][tx], acc);
    __syncthreads();
  }
  const int m = m0 + ty, n = n0 + tx;
  if (m < M && n < d) Y[(int64_t)m * d + n] = acc;
}

// I = 0 for an empty prompt (every column norm is 0).
__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------- host
static int z_pitch(int32_t d_ff) { return (int)align_up((size_t)d_ff, kZPad); }

static size_t prompt_ffn_ws_bytes(int64_t n_tokens, int32_t d_ff, int e) {
  const int64_t rows = n_tokens < kChunkTokens ? n_tokens : kChunkTokens;
  return align_up((size_t)align_up((size_t)rows, kBM) * (size_t)z_pitch(d_ff) * (size_t)e, 256);
}

static pop_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}

// With s2 and I set, the first chunk's gate/up launch also writes I.
static void launch_prompt_ffn(hipStream_t st, const void* X, int64_t n_tokens, int32_t d, const void* Wg,
                              const void* Wu, const void* WdT, int32_t d_ff, pop_dtype dt, float* Y, void* ws,
                              const float* s2 = nullptr, float* I = nullptr) {
  const int ldz = z_pitch(d_ff);
  for (int64_t t0 = 0; t0 < n_tokens; t0 += kChunkTokens) {
    const int M = (int)(n_tokens - t0 < kChunkTokens ? n_tokens - t0 : kChunkTokens);
    float* Yc = Y + t0 * d;
    const bool imp = I != nullptr && t0 == 0;
    if (dt == POP_BF16) {
      const bf16s* Xc = (const bf16s*)X + t0 * d;
      const int mt = (M + kBM - 1) / kBM;
      const int nt1 = ldz / kBN;
      if (imp && mt >= 4)
        POP_LAUNCH((k_prompt_gateup<16, POP_GATEUP_NS>), dim3(mt * nt1), dim3(kGThreads), 0, st, Xc, M, (int)d, (const bf16s*)Wg,
                   (const bf16s*)Wu, (int)d_ff, (uint16_t*)ws, ldz, mt, nt1, s2, I);
      else if (imp)
        POP_LAUNCH((k_prompt_gateup<64, POP_GATEUP_NS>), dim3(mt * nt1), dim3(kGThreads), 0, st, Xc, M, (int)d, (const bf16s*)Wg,
                   (const bf16s*)Wu, (int)d_ff, (uint16_t*)ws, ldz, mt, nt1, s2, I);
      else
        POP_LAUNCH((k_prompt_gateup<0, POP_GATEUP_NS>), dim3(mt * nt1), dim3(kGThreads), 0, st, Xc, M, (int)d, (const bf16s*)Wg,
                   (const bf16s*)Wu, (int)d_ff, (uint16_t*)ws, ldz, mt, nt1, (const float*)nullptr, (float*)nullptr);
      const int nt2 = (d + kBN - 1) / kBN;
      // short prompts: 64-token tiles, for twice the blocks (a block's K loop is latency-bound)
      const int mt64 = (M + 63) / 64;
      if (mt * nt2 < POP_DOWN_BM64_BELOW)
        POP_LAUNCH((k_prompt_down<64, POP_DOWN_NS>), dim3(mt64 * nt2), dim3(kGThreads), 0, st, (const uint16_t*)ws,
                   M, ldz, (const bf16s*)WdT, (int)d_ff, (int)d, Yc, mt64, nt2);
      else
        POP_LAUNCH((k_prompt_down<128, POP_DOWN_NS>), dim3(mt * nt2), dim3(kGThreads), 0, st, (const uint16_t*)ws,
                   M, ldz, (const bf16s*)WdT, (int)d_ff, (int)d, Yc, mt, nt2);
    } else {
      const float* Xc = (const float*)X + t0 * d;
      const int mt = (M + kFT - 1) / kFT;
      if (imp)
        POP_LAUNCH(k_prompt_gateup_f32<true>, dim3((d_ff + kFT - 1) / kFT, mt), dim3(kFT * kFT), 0, st, Xc, M,
                   (int)d, (const float*)Wg, (const float*)Wu, (int)d_ff, (float*)ws, ldz, s2, I);
      else
        POP_LAUNCH(k_prompt_gateup_f32<false>, dim3((d_ff + kFT - 1) / kFT, mt), dim3(kFT * kFT), 0, st, Xc, M,
                   (int)d, (const float*)Wg, (const float*)Wu, (int)d_ff, (float*)ws, ldz, (const float*)nullptr,
                   (float*)nullptr);
      POP_LAUNCH(k_prompt_down_f32, dim3((d + kFT - 1) / kFT, mt), dim3(kFT * kFT), 0, st, (const float*)ws, M,
                 ldz, (const float*)WdT, (int)d_ff, (int)d, Yc);
    }
  }
}

void launch_gemm_kmajor(void* stream, const void* A, int M, int lda, const void* Bk, int K, int N, pop_dtype dt,
                        float* Y) {
  hipStream_t st = (hipStream_t)stream;
  for (int m0 = 0; m0 < M; m0 += (int)kChunkTokens) {  // row chunks keep every grid dimension small
    const int Mc = M - m0 < (int)kChunkTokens ? M - m0 : (int)kChunkTokens;
    float* Yc = Y + (int64_t)m0 * N;
    if (dt == POP_BF16) {
      const int mt = (Mc + kBM - 1) / kBM, nt = (N + kBN - 1) / kBN;
      POP_LAUNCH((k_prompt_down<128, POP_DOWN_NS>), dim3(mt * nt), dim3(kGThreads), 0, st,
                 (const uint16_t*)A + (int64_t)m0 * lda, Mc, lda, (const bf16s*)Bk, K, N, Yc, mt, nt);
    } else {
      POP_LAUNCH(k_prompt_down_f32, dim3((N + kFT - 1) / kFT, (Mc + kFT - 1) / kFT), dim3(kFT * kFT), 0, st,
                 (const float*)A + (int64_t)m0 * lda, Mc, lda, (const float*)Bk, K, N, Yc);
    }
  }
}

}  // namespace pop

using namespace pop;

extern "C" size_t pop_dense_ffn_prefill_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff, pop_dtype dt) {
  if (n_tokens < 0 || d <= 0 || d_ff <= 0 || (dt != POP_BF16 && dt != POP_F32)) return 0;
  return prompt_ffn_ws_bytes(n_tokens, d_ff, elem_bytes(dt));
}

// Fused prefill: column norms, then the prompt FFN whose gate/up pass also
// yields the importance, then the partition.  Workspace: the Z buffer, the
// column-norm workspace, and I when the caller passes none.
static size_t fused_prefill_ws_bytes(int64_t n_tokens, int32_t d, int32_t d_ff, pop_dtype dt) {
  return prompt_ffn_ws_bytes(n_tokens, d_ff, elem_bytes(dt)) + colsq_ws_bytes(n_tokens, d) +
         align_up((size_t)d_ff * sizeof(float), 256);
}

extern "C" size_t pop_prefill_ffn_partition_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff, pop_dtype dt) {
  if (n_tokens < 0 || d <= 0 || d_ff <= 0 || (dt != POP_BF16 && dt != POP_F32)) return 0;
  return fused_prefill_ws_bytes(n_tokens, d, d_ff, dt);
}

extern "C" pop_status pop_prefill_ffn_partition(const void* X, int64_t n_tokens, int32_t d, const void* W_gate,
                                                const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                                double r, double gamma, float* Y, int32_t* R, int32_t* C, int32_t* P,
                                                float* importance, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_dtype_width(dt, d);
  if (s != POP_OK) return s;
  if ((s = check_rate(r, gamma)) != POP_OK) return s;
  if (d > POP_MAX_D) return fail(POP_ERR_BAD_SHAPE, "d=%d above %d", d, POP_MAX_D);
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (n_tokens < 0 || n_tokens > ((int64_t)1 << 40) / d)
    return fail(POP_ERR_BAD_SHAPE, "n_tokens=%lld out of range", (long long)n_tokens);
  if (W_gate == nullptr || W_up == nullptr || W_downT == nullptr || ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "W_gate, W_up, W_downT and ws must be non-NULL");
  if (n_tokens > 0 && (X == nullptr || Y == nullptr))
    return fail(POP_ERR_INVALID_ARGUMENT, "X and Y must be non-NULL when n_tokens > 0");
  const pop_counts c = counts(d_ff, r, gamma);
  if ((c.n_R > 0 && R == nullptr) || (c.n_C > 0 && C == nullptr) || (c.n_P > 0 && P == nullptr))
    return fail(POP_ERR_INVALID_ARGUMENT, "an output list with a nonzero size is NULL");
  if (!aligned16(X) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_downT) || !aligned16(Y) ||
      !aligned16(ws) || !aligned16(importance))
    return fail(POP_ERR_MISALIGNED, "buffers must be 16-byte aligned");
  const size_t need = fused_prefill_ws_bytes(n_tokens, d, d_ff, dt);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  char* base = (char*)ws;
  char* zws = base;
  char* cws = zws + prompt_ffn_ws_bytes(n_tokens, d_ff, elem_bytes(dt));
  float* I = importance ? importance : (float*)(cws + colsq_ws_bytes(n_tokens, d));
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  const float* s2 = launch_colsq(st, X, n_tokens, d, dt, cws);
  if (n_tokens > 0)
    launch_prompt_ffn(st, X, n_tokens, d, W_gate, W_up, W_downT, d_ff, dt, Y, zws, s2, I);
  else
    POP_LAUNCH(k_zero_f32, dim3((d_ff + 255) / 256), dim3(256), 0, st, I, (int)d_ff);
  launch_partition_lists(st, I, d_ff, c.c_low, c.c_high, R, C, P);
  return launched();
}

extern "C" pop_status pop_dense_ffn_prefill(const void* X, int64_t n_tokens, int32_t d, const void* W_gate,
                                            const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                            float* Y, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_dtype_width(dt, d);
  if (s != POP_OK) return s;
  if (d > POP_MAX_D) return fail(POP_ERR_BAD_SHAPE, "d=%d above %d", d, POP_MAX_D);
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (n_tokens < 0 || n_tokens > ((int64_t)1 << 40) / d)
    return fail(POP_ERR_BAD_SHAPE, "n_tokens=%lld out of range", (long long)n_tokens);
  if (W_gate == nullptr || W_up == nullptr || W_downT == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "W_gate, W_up and W_downT must be non-NULL");
  if (n_tokens > 0 && (X == nullptr || Y == nullptr || ws == nullptr))
    return fail(POP_ERR_INVALID_ARGUMENT, "X, Y and ws must be non-NULL when n_tokens > 0");
  if (!aligned16(X) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_downT) || !aligned16(Y) ||
      !aligned16(ws))
    return fail(POP_ERR_MISALIGNED, "buffers must be 16-byte aligned");
  const size_t need = prompt_ffn_ws_bytes(n_tokens, d_ff, elem_bytes(dt));
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  launch_prompt_ffn(st, X, n_tokens, d, W_gate, W_up, W_downT, d_ff, dt, Y, ws);
  return launched();
}
