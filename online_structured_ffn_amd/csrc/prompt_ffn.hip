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
// Both bf16 GEMMs run one 256-thread workgroup per compute unit, each with a
// ring of stages in LDS that direct-to-LDS loads (global_load_lds_dwordx4)
// fill several stages ahead of the matrix cores, so no operand passes through
// registers on its way in.  Operand tiles sit in LDS K-contiguous (X, W_gate,
// W_up and Z rows) or N-contiguous (W_downT rows, [d_ff, d], read back with
// the transposing LDS read ds_read_b64_tr_b16), their 16- or 32-byte units
// XOR-swizzled so that both the loads' 1 KB writes and the fragment reads
// stay free of bank conflicts.
#include <hip/hip_runtime.h>

#include <utility>

#include "pop_device.h"
#include "pop_internal.h"
#include "prompt_gemm.h"

namespace pop {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaveThreads = 256;  // one group of four waves
constexpr int kBM = 128;         // tokens per block (both GEMMs): 32 per wave of a group
constexpr int kDnKC = 64;        // down: reduction elements per stage
constexpr int kDnBN = 64;        // down: output columns per block
constexpr int kZPad = 64;        // Z row pitch = d_ff rounded up to this
constexpr int64_t kChunkTokens = 4096;  // tokens per pass (bounds the workspace)
#ifndef POP_PROMPT_GR
#define POP_PROMPT_GR 1  // groups of four waves per workgroup (1 or 2), taking alternating stages
#endif
#ifndef POP_GATEUP_NS
#define POP_GATEUP_NS 5  // stages in the gate/up LDS ring (a multiple of the group count)
#endif
#ifndef POP_DOWN_NS
#define POP_DOWN_NS 6  // stages in the down-projection LDS ring (a multiple of the group count)
#endif
#ifndef POP_GATEUP_PD
#define POP_GATEUP_PD 2  // channel fragments read ahead of the MFMAs in the gate/up pass
#endif
constexpr int kGuThreads = kWaveThreads * POP_PROMPT_GR;  // threads per workgroup (one per compute unit)
#ifndef POP_GATEUP_KC
#define POP_GATEUP_KC 32  // gate/up: reduction elements per stage (32: 64-byte rows, 64: 128-byte rows)
#endif
constexpr int kGuKC = POP_GATEUP_KC;

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One direct-to-LDS load of a wave: lane i's 16 bytes at g land at LDS byte
// address lds + 16 i (lds wave-uniform).  Written out rather than taken from
// the builtin: the compiler makes LDS reads (the transposing read among them)
// wait for every builtin direct-to-LDS load in flight, which would drain the
// ring at each stage.  The loads write no register; the ring's own waits
// (ring_barrier) account for them.  M0 carries the LDS address; nothing else
// in these kernels uses M0 (LDS reads on gfx950 do not), so the clobber only
// records that the statement sets it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Waits until at most N vector-memory instructions of this wave are in
// flight and every LDS access of the wave is done, then a workgroup barrier.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16 zero bytes: the source of every operand chunk past the reduction's end.
__device__ __align__(16) const uint32_t kZero16[4] = {0u, 0u, 0u, 0u};


// K-contiguous tiles in LDS: rows of KC elements (KC = 32: 64 bytes, KC = 64:
// 128 bytes), 16-byte chunk c of row r in slot kslot<KC>(c, r) of the row.
// With these swizzles the fragment reads (16 rows, one chunk each, per 16-lane
// group) run without LDS bank conflicts, measured with the bank-conflict
// counter (4 LDS cycles per 64-lane 16-byte read; the swizzle c ^ ((r >> 2) &
// 3) of 64-byte rows takes 8), and one wave's direct-to-LDS load fills whole
// rows.
template <int KC>
__device__ __forceinline__ int kslot(int c, int r) {
  if constexpr (KC == 32)
    return c ^ ((r >> 1) & 3);
  else
    return c ^ ((r >> 1) & 7);
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
// Block tile: 128 tokens x 16 NF channels of each matrix.  A stage holds 32
// reduction columns of the 128 token rows, then the 16 NF gate rows, then the
// 16 NF up rows (64 bytes each, K-contiguous).  The eight waves form two
// groups of four; group g computes the stages of parity g, so two waves share
// each SIMD and one's MFMAs run while the other waits.  Wave w of a group
// computes tokens 32 w + [0, 32) against every channel of the block (2 x NF
// fragments per matrix) over its group's stages; at the end group 1 adds its
// sums into group 0's through LDS (group 0 + group 1, a fixed order).  NF is
// chosen at launch so that the tiles fill the compute units in as few rounds
// as possible.
//
// IMP > 0: the first IMP token tiles' blocks also compute the importance
// I_i = sqrt(sum_k W_up[i,k]^2 * s2[k]) of the block's channels from the W_up
// rows already in LDS (the column norms s2 of the whole prompt are an input),
// so the prefill needs no second sweep of W_up.  Block m_tile takes channels
// m_tile * G + [0, G), G = 16 NF / IMP; wave w of group g sums columns 8 w +
// [0, 8) of its group's stages (in ascending order) for channel lane + 64 j,
// with s2 from scalar loads; the eight partial sums of a channel are added in
// (group, wave) order.
//
// Ring of NS stages (NS even): stages 0 .. NS - 3 load first; step j waits for
// the wave's own loads of stages 2 j and 2 j + 1, passes a barrier (every
// wave's share landed, both groups done with stages 2 j - 2 and 2 j - 1),
// then group g computes stage 2 j + g while every wave issues its share of
// stages 2 j + NS - 2 and 2 j + NS - 1 into the freed slots.  Stages past the
// last one (at most one, when the count is odd, and the refills past the end)
// load zeros.  Rows past M and channels past d_ff load clamped rows (their
// outputs are not written, or written as 0); chunks past d load zeros.
template <int NF, int NS, int IMP, int GR>
__global__ __launch_bounds__(kWaveThreads * GR, 1) void k_prompt_gateup(const bf16s* __restrict__ X, int M, int d,
                                                                const bf16s* __restrict__ Wg,
                                                                const bf16s* __restrict__ Wu, int d_ff,
                                                                uint16_t* __restrict__ Z, int ldz, int mt, int nt,
                                                                const float* __restrict__ s2, float* __restrict__ I) {
  constexpr int KC = kGuKC;
  constexpr int CPR = KC / 8;            // 16-byte chunks per row and stage
  constexpr int RPI = 64 / CPR;          // rows per load instruction (1 KB)
  constexpr int KH = KC / 32;            // 32-reduction halves per stage
  constexpr int BR = 16 * NF;            // channels per block and matrix
  constexpr int ROWS = kBM + 2 * BR;     // tile rows per stage
  constexpr int NI = ROWS / RPI;         // load instructions per stage
  constexpr int NW = 4 * GR;             // waves
  constexpr int LPW = (NI + NW - 1) / NW;  // per wave; the spare ones repeat instruction NI - 1
  constexpr int STILE = ROWS * KC;       // bf16 elements of a stage's tile
  constexpr int STAGE = STILE + (IMP > 0 ? 512 : 0);   // + 1 KB holding the stage's s^2 (importance only)
  constexpr int NSF = 163840 / (2 * STAGE) / GR * GR;  // stages that fit in LDS
  constexpr int NSR = NS < NSF ? NS : NSF;             // ring depth
  constexpr int G = IMP > 0 ? BR / (IMP > 0 ? IMP : 1) : 1;  // importance channels per block
  constexpr int NPR = (G + 63) / 64;
  static_assert(KC == 32 || KC == 64, "stage width");
  static_assert(NSR % GR == 0 && NSR >= 2 * GR && (NSR - 2 * GR) * LPW < 64, "ring depth");
  static_assert(GR * LPW <= KH * NF, "the refill loads ride on the first GR LPW fragment steps");
  __shared__ __align__(16) uint16_t smem[NSR * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wv = wave & 3;
  int m_tile, n_tile;
  tile_of(blockIdx.x, mt * nt, mt, m_tile, n_tile);
  const int m0 = m_tile * kBM, n0 = n_tile * BR;
  const uint32_t lds0 = lds_addr(smem);

  // load instruction m of this wave fills rows RPI j + [0, RPI): lane i row
  // RPI j + i / CPR, slot i % CPR, which holds chunk co[m] / 8 of that row
  const bf16s* rowp[LPW];
  int co[LPW];
  uint32_t lofs[LPW];
#pragma unroll
  for (int m = 0; m < LPW; ++m) {
    const int j = min(wave + NW * m, NI - 1);
    const int row = RPI * j + lane / CPR;
    const bf16s* p;
    if (row < kBM)
      p = X + (int64_t)min(m0 + row, M - 1) * d;
    else if (row < kBM + BR)
      p = Wg + (int64_t)min(n0 + row - kBM, d_ff - 1) * d;
    else
      p = Wu + (int64_t)min(n0 + row - kBM - BR, d_ff - 1) * d;
    rowp[m] = p;
    co[m] = 8 * kslot<KC>(lane % CPR, row);
    lofs[m] = 2u * RPI * KC * j;
  }
  // load m of stage st into ring slot q; m = LPW (wave 0, importance only):
  // the stage's KC values of s^2, 16 bytes a lane (lanes past them load zeros)
  auto issue1 = [&](int st, int q, int m) {
    const int k0 = st * KC;
    if (m < LPW)
      dma16(k0 + co[m] < d ? (const void*)(rowp[m] + k0 + co[m]) : (const void*)kZero16,
            lds0 + 2u * STAGE * q + lofs[m]);
    else if (IMP > 0 && wave == 0)
      dma16(lane < KC / 4 && k0 + 4 * lane < d ? (const void*)(s2 + k0 + 4 * lane) : (const void*)kZero16,
            lds0 + 2u * (STAGE * q + STILE));
  };

  const bool imp = IMP > 0 && m_tile < IMP;  // block-uniform
  float ia[NPR];
#pragma unroll
  for (int j = 0; j < NPR; ++j) ia[j] = 0.f;

  f32x4 ag[2][NF], au[2][NF];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) ag[i][f] = au[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15;
  // Stage st from slot q, as NX = KH NF fragment steps x = h NF + f (half h,
  // channel fragment f); the reads run PD steps ahead of the MFMAs, and the
  // refill (stages rst .. rst + GR - 1 into slots rq .., this wave's share)
  // rides on the first steps, one load each; the scheduling barriers keep
  // that order.
  auto compute = [&](int st, int q, int rst, int rq) {
    const uint16_t* base = smem + q * STAGE;
    constexpr int NX = KH * NF;
    constexpr int PD = POP_GATEUP_PD < NX ? POP_GATEUP_PD : NX;
    bf16x8 a[KH][2], bg[NX], bu[NX];
    auto read_a = [&](int h) {
      const int sl = 8 * kslot<KC>(4 * h + (lane >> 4), fr);
#pragma unroll
      for (int i = 0; i < 2; ++i) a[h][i] = lds_frag(base + (32 * wv + 16 * i + fr) * KC + sl);
    };
    auto read_b = [&](int x) {
      const int h = x / NF, f = x % NF;
      const int sl = 8 * kslot<KC>(4 * h + (lane >> 4), fr);
      bg[x] = lds_frag(base + (kBM + 16 * f + fr) * KC + sl);
      bu[x] = lds_frag(base + (kBM + BR + 16 * f + fr) * KC + sl);
    };
    // Importance (IMP > 0): per chunk h (columns 8 (wv + 4 h) + [0, 8)) one
    // read of the W_up row of channel m_tile G + lane + 64 j and of the
    // chunk's s^2 (the same 32 bytes for every lane), then four steps of two
    // products each, spread over the last fragment steps so that they run
    // between the MFMAs.  Every block does it (the blocks past the first IMP
    // token tiles and the lanes past G compute sums that are never stored);
    // chunks past d hold zeros.
    u32x4 wi[KH][NPR];
    f32x4 sv[KH][2];
    constexpr int NK = 5 * KH;  // importance steps
    auto imp_step = [&](int k) {
      const int h = k / 5, s = k % 5;
      if (s == 0) {
        const f32x4* sp = reinterpret_cast<const f32x4*>(base + STILE) + 2 * (wv + 4 * h);
        sv[h][0] = sp[0];
        sv[h][1] = sp[1];
#pragma unroll
        for (int j = 0; j < NPR; ++j) {
          const int row = kBM + BR + m_tile * G + min(lane + 64 * j, G - 1);
          wi[h][j] = *reinterpret_cast<const u32x4*>(base + row * KC + 8 * kslot<KC>(wv + 4 * h, row));
        }
      } else {
        const int e = s - 1;
#pragma unroll
        for (int j = 0; j < NPR; ++j) {
          const float w0 = __uint_as_float(wi[h][j][e] << 16), w1 = __uint_as_float(wi[h][j][e] & 0xffff0000u);
          ia[j] = fmaf(w0 * w0, sv[h][e >> 1][2 * (e & 1)], ia[j]);
          ia[j] = fmaf(w1 * w1, sv[h][e >> 1][2 * (e & 1) + 1], ia[j]);
        }
      }
    };
    read_a(0);
#pragma unroll
    for (int x = 0; x < PD; ++x) {
      if (x > 0 && x % NF == 0) read_a(x / NF);
      read_b(x);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int y = x + PD;
      if (y < NX) {
        if (y % NF == 0) read_a(y / NF);
        read_b(y);
      }
      if (x < GR * LPW) issue1(rst + x / LPW, rq + x / LPW, x % LPW);
      if (IMP > 0 && x == (GR * LPW < NX ? GR * LPW : NX - 1))
#pragma unroll
        for (int r = 0; r < GR; ++r) issue1(rst + r, rq + r, LPW);
      if constexpr (IMP > 0) {
#pragma unroll
        for (int k = 0; k < NK; ++k)
          if ((NX >= NK ? NX - NK + k : k * NX / NK) == x) imp_step(k);
      }
      const int h = x / NF, f = x % NF;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ag[i][f] = mfma(a[h][i], bg[x], ag[i][f]);
        au[i][f] = mfma(a[h][i], bu[x], au[i][f]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // (the inner loop unrolls fully: every ring slot index is a constant)
  const int nst = (d + KC - 1) / KC;
#pragma unroll
  for (int u = 0; u < NSR - GR; ++u)
#pragma unroll
    for (int m = 0; m < LPW + (IMP > 0 ? 1 : 0); ++m) issue1(u, u, m);
  for (int s0 = 0; s0 < nst; s0 += NSR) {
#pragma unroll
    for (int u = 0; u < NSR; u += GR) {
      const int st = s0 + u;
      if (st >= nst) break;
      ring_barrier<(NSR - 2 * GR) * LPW>();
      compute(st + grp, u + grp, st + NSR - GR, (u + NSR - GR) % NSR);
    }
  }
  ring_barrier<0>();  // the spare loads landed; every wave is done with the ring

  // group 1's sums into group 0's, in two rounds of fragments
  float* red = reinterpret_cast<float*>(smem);
  constexpr int NH = (NF + 1) / 2;
#pragma unroll
  for (int r = 0; r < (GR > 1 ? 2 : 0); ++r) {
    const int f0 = r == 0 ? 0 : NH, f1 = r == 0 ? NH : NF;
    float* rw = red + wv * (2 * NH * 2 * 4) * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int f = f0; f < f1; ++f)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            rw[(((f - f0) * 2 + i) * 8 + e) * 64] = ag[i][f][e];
            rw[(((f - f0) * 2 + i) * 8 + 4 + e) * 64] = au[i][f][e];
          }
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
      for (int f = f0; f < f1; ++f)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ag[i][f][e] += rw[(((f - f0) * 2 + i) * 8 + e) * 64];
            au[i][f][e] += rw[(((f - f0) * 2 + i) * 8 + 4 + e) * 64];
          }
    }
    __syncthreads();
  }
  if (imp) {  // block-uniform
#pragma unroll
    for (int j = 0; j < NPR; ++j)
      if (lane + 64 * j < G) red[wave * G + lane + 64 * j] = ia[j];
    __syncthreads();
    for (int c = tid; c < G; c += NW * 64) {
      const int ch = n0 + m_tile * G + c;
      float t = red[c];
#pragma unroll
      for (int w = 1; w < NW; ++w) t += red[w * G + c];
      if (ch < d_ff) I[ch] = sqrtf(t);
    }
  }
  if (grp != 0) return;
  // Output fragment layout: element e of lane l is row (l >> 4) * 4 + e,
  // column l & 15 of the 16 x 16 tile.  Columns in [d_ff, ldz) are written as
  // 0: Z's padding must be zero for the second GEMM.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = n0 + 16 * f + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 32 * wv + 16 * i + (lane >> 4) * 4 + e;
        if (m < M && n < ldz)
          Z[(int64_t)m * ldz + n] = n < d_ff ? bf16_rne(silu(ag[i][f][e]) * au[i][f][e]) : (uint16_t)0;
      }
    }
}

// ---------------------------------------------------------------- down
// Y[m, n] = sum_k A[m, k] Bk[k, n] (the prompt FFN: A = Z, Bk = W_downT).
// Block tile: 128 tokens x 64 columns; a stage holds 64 reduction columns of
// the 128 A rows (K-contiguous, 128 bytes a row) and the 64 Bk rows of those
// reductions (N-contiguous, 128 bytes a row).  The Bk tile is read with the
// transposing LDS read: within a 16-lane group, lane i receives element i % 4
// of the 8 bytes addressed by lanes 4 e + i / 4, e = 0 .. 3; the lanes of
// group g address rows 8 g + [0, 4) (then 8 g + 4 + [0, 4)), four lanes per
// row, 4 columns each, which hands every lane the 8 consecutive reductions of
// one column that the MFMA operand holds.  The 32-byte column units of Bk row
// r are stored XOR-ed with bsw(r), which keeps the rows that one transposing
// read touches on distinct banks.  Two groups of four waves take alternating
// stages as in the gate/up pass; wave w of a group computes tokens 32 w +
// [0, 32) x all 64 columns (2 x 4 fragments), and group 1's sums join group
// 0's through LDS at the end.
//
// Ka: A's reduction extent (a multiple of 8; chunks past it load zeros); Kb:
// Bk's rows (rows past it load clamped rows, which meet those zeros or A's zero
// padding).  Rows past M and columns past N load clamped data and are not
// written.  The ring works as in the gate/up pass.
__device__ __forceinline__ int bsw(int r) { return ((r >> 1) & 1) | ((r >> 2) & 2); }

__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* p, int second) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + second));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int NS, int GR>
__global__ __launch_bounds__(kWaveThreads * GR, 1) void k_prompt_down(const uint16_t* __restrict__ A, int M, int lda, int Ka,
                                                              const bf16s* __restrict__ Bk, int Kb, int N,
                                                              float* __restrict__ Y, int mt, int nt) {
  constexpr int KC = kDnKC, BN = kDnBN;
  constexpr int NIA = kBM * KC / 512;    // A load instructions per stage (8 rows of 128 bytes each)
  constexpr int NIB = KC * BN / 512;     // Bk load instructions per stage
  constexpr int NW = 4 * GR;             // waves
  constexpr int LA = NIA / NW, LB = NIB / NW;
  constexpr int NV = LA + LB;            // load instructions per stage and wave
  constexpr int ASZ = kBM * KC;          // bf16 elements of the A part
  constexpr int STAGE = ASZ + KC * BN;
  static_assert(KC == 64 && BN == 64, "the transposing reads' offsets assume 64 x 64 Bk tiles");
  static_assert(NIA % NW == 0 && NIB % NW == 0, "load shares");
  static_assert(NS % GR == 0 && NS >= 2 * GR && (NS - 2 * GR) * NV < 64, "ring depth");
  static_assert(GR * NV <= 8, "the refill loads ride on the first GR NV fragment pairs");
  __shared__ __align__(16) uint16_t smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wv = wave & 3;
  int m_tile, n_tile;
  tile_of(blockIdx.x, mt * nt, mt, m_tile, n_tile);
  const int m0 = m_tile * kBM, n0 = n_tile * BN;
  const bf16s* Ab = reinterpret_cast<const bf16s*>(A);
  const uint32_t lds0 = lds_addr(smem);

  // A: instruction j fills rows 8 j + [0, 8): lane i row 8 j + i / 8, slot i % 8
  const bf16s* arow[LA];
  int aco[LA];
#pragma unroll
  for (int m = 0; m < LA; ++m) {
    const int j = wave + NW * m;
    const int row = 8 * j + (lane >> 3);
    arow[m] = Ab + (int64_t)min(m0 + row, M - 1) * lda;
    aco[m] = 8 * ((lane & 7) ^ (((j & 1) << 2) | (lane >> 4)));
  }
  // Bk: instruction j fills rows 8 j + [0, 8): lane i row r = 8 j + i / 8,
  // bytes 16 (i % 8) of it, i.e. half i % 2 of physical unit (i % 8) / 2
  int bro[LB], bco[LB];
#pragma unroll
  for (int m = 0; m < LB; ++m) {
    const int j = wave + NW * m;
    const int r = 8 * j + (lane >> 3);
    const int u = ((lane & 7) >> 1) ^ bsw(r);
    bro[m] = r;
    bco[m] = min(n0 + 16 * u + 8 * (lane & 1), N - 8);
  }
  // load m of stage st into ring slot q (m < LA: A, else Bk)
  auto issue1 = [&](int st, int q, int m) {
    const int k0 = st * KC;
    const uint32_t base = lds0 + 2u * STAGE * q;
    if (m < LA)
      dma16(k0 + aco[m] < Ka ? (const void*)(arow[m] + k0 + aco[m]) : (const void*)kZero16,
            base + 2u * (8 * (wave + NW * m) * KC));
    else
      dma16(Bk + (int64_t)min(k0 + bro[m - LA], Kb - 1) * N + bco[m - LA],
            base + 2u * (ASZ + 8 * (wave + NW * (m - LA)) * BN));
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, g = lane >> 4;
  // transposing reads: this lane addresses row 8 g + (fr >> 2) (+ 4) of each
  // 32-reduction half, columns 4 (fr & 3) of the fragment's unit
  const int trow = 8 * g + (fr >> 2);
  const int tsw = bsw(trow);
  // Stage st from slot q: every read first (the second half's land under the
  // first half's MFMAs), then per (half, fragment) one refill load (stages rst
  // and rst + 1 into slots rq and rq + 1, this wave's share) and 2 MFMAs.
  auto compute = [&](int st, int q, int rst, int rq) {
    const uint16_t* base = smem + q * STAGE;
    bf16x8 a[2][2], b[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 4 * h + g;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * wv + 16 * i + fr;
        a[h][i] = lds_frag(base + row * KC + 8 * kslot<KC>(c, row));
      }
#pragma unroll
      for (int f = 0; f < 4; ++f)
        b[h][f] = tr_frag(base + ASZ + (32 * h + trow) * BN + 16 * (f ^ tsw) + 4 * (fr & 3), 4 * BN);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int p = 4 * h + f;
        if (p < GR * NV) issue1(rst + p / NV, rq + p / NV, p % NV);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][f] = mfma(a[h][i], b[h][f], acc[i][f]);
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // (the inner loop unrolls fully: every ring slot index is a constant)
  const int nst = (Ka + KC - 1) / KC;
#pragma unroll
  for (int u = 0; u < NS - GR; ++u)
#pragma unroll
    for (int m = 0; m < NV; ++m) issue1(u, u, m);
  for (int s0 = 0; s0 < nst; s0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; u += GR) {
      const int st = s0 + u;
      if (st >= nst) break;
      ring_barrier<(NS - 2 * GR) * NV>();
      compute(st + grp, u + grp, st + NS - GR, (u + NS - GR) % NS);
    }
  }
  ring_barrier<0>();
  float* red = reinterpret_cast<float*>(smem) + wv * 32 * 64 + lane;
  if (GR > 1 && grp == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((i * 4 + f) * 4 + e) * 64] = acc[i][f][e];
  }
  __syncthreads();
  if (grp != 0) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int n = n0 + 16 * f + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 32 * wv + 16 * i + 4 * g + e;
        if (m < M && n < N) Y[(int64_t)m * N + n] = GR > 1 ? acc[i][f][e] + red[((i * 4 + f) * 4 + e) * 64] : acc[i][f][e];
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

// Gate/up block shape.  NF (channel fragments per block and matrix) is picked
// per launch: the mt x ceil(ldz / 16 NF) tiles run in ceil(tiles / slots)
// rounds on slots = compute units x resident blocks per unit, and a round
// costs about (NF + 1) x (resident blocks per unit) units of one unit's time
// (NF fragments of the weights plus the token operand).  The least total wins;
// ties go to the larger NF (fewer re-reads of the prompt).
template <int NF, int IMP>
static const void* gateup_kernel() {
  return reinterpret_cast<const void*>(&k_prompt_gateup<NF, POP_GATEUP_NS, IMP, POP_PROMPT_GR>);
}
template <int NF>
static const void* gateup_kernel_imp(int imp) {
  return imp == 4 ? gateup_kernel<NF, 4>() : imp == 2 ? gateup_kernel<NF, 2>() : imp == 1 ? gateup_kernel<NF, 1>()
                                                                                          : gateup_kernel<NF, 0>();
}
static const void* gateup_kernel_of(int nf, int imp) {
  switch (nf) {
    case 4: return gateup_kernel_imp<4>(imp);
    case 6: return gateup_kernel_imp<6>(imp);
    case 8: return gateup_kernel_imp<8>(imp);
    case 10: return gateup_kernel_imp<10>(imp);
    default: return gateup_kernel_imp<11>(imp);
  }
}
constexpr int kGateupNF[] = {4, 6, 8, 10, 11};

struct GateupShape {
  int n_cu = 0;
  int per_cu[5] = {};  // resident blocks per compute unit, by kGateupNF entry
};
static const GateupShape& gateup_shape() {
  static GateupShape sh[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!done[dev]) {
    GateupShape s;
    if (hipDeviceGetAttribute(&s.n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || s.n_cu < 1)
      s.n_cu = 256;
    for (int i = 0; i < 5; ++i) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, gateup_kernel_of(kGateupNF[i], 0), kGuThreads, 0) !=
              hipSuccess ||
          nb < 1)
        nb = 1;
      s.per_cu[i] = nb;
    }
    sh[dev] = s;
    done[dev] = true;
  }
  return sh[dev];
}
static int gateup_nf(int mt, int ldz) {
  const GateupShape& s = gateup_shape();
  int best = 11;
  int64_t best_cost = -1;
  for (int i = 0; i < 5; ++i) {
    const int nf = kGateupNF[i];
    const int64_t tiles = (int64_t)mt * ((ldz + 16 * nf - 1) / (16 * nf));
    const int64_t slots = (int64_t)s.n_cu * s.per_cu[i];
    const int64_t cost = (tiles + slots - 1) / slots * (nf + 1) * s.per_cu[i];
    if (best_cost < 0 || cost <= best_cost) best = nf, best_cost = cost;
  }
  return best;
}

template <int NF>
static void launch_gateup_nf(hipStream_t st, int imp, const bf16s* X, int M, int d, const bf16s* Wg,
                             const bf16s* Wu, int d_ff, uint16_t* Z, int ldz, int mt, const float* s2, float* I) {
  const int nt = (ldz + 16 * NF - 1) / (16 * NF);
  const dim3 grid(mt * nt), block(kGuThreads);
  if (imp == 4)
    POP_LAUNCH((k_prompt_gateup<NF, POP_GATEUP_NS, 4, POP_PROMPT_GR>), grid, block, 0, st, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, nt, s2, I);
  else if (imp == 2)
    POP_LAUNCH((k_prompt_gateup<NF, POP_GATEUP_NS, 2, POP_PROMPT_GR>), grid, block, 0, st, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, nt, s2, I);
  else if (imp == 1)
    POP_LAUNCH((k_prompt_gateup<NF, POP_GATEUP_NS, 1, POP_PROMPT_GR>), grid, block, 0, st, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, nt, s2, I);
  else
    POP_LAUNCH((k_prompt_gateup<NF, POP_GATEUP_NS, 0, POP_PROMPT_GR>), grid, block, 0, st, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, nt,
               (const float*)nullptr, (float*)nullptr);
}

// Z = SiLU(X W_gate^T) * (X W_up^T) for M <= kChunkTokens tokens; with imp > 0
// (the number of token tiles, 1, 2 or 4, that share the work) the launch also
// writes I from s2.
static void launch_gateup(hipStream_t st, int imp, const bf16s* X, int M, int d, const bf16s* Wg, const bf16s* Wu,
                          int d_ff, uint16_t* Z, int ldz, const float* s2, float* I) {
  const int mt = (M + kBM - 1) / kBM;
  switch (gateup_nf(mt, ldz)) {
    case 4: launch_gateup_nf<4>(st, imp, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, s2, I); break;
    case 6: launch_gateup_nf<6>(st, imp, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, s2, I); break;
    case 8: launch_gateup_nf<8>(st, imp, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, s2, I); break;
    case 10: launch_gateup_nf<10>(st, imp, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, s2, I); break;
    default: launch_gateup_nf<11>(st, imp, X, M, d, Wg, Wu, d_ff, Z, ldz, mt, s2, I); break;
  }
}

// Y [M, N] = A [M, Ka] (pitch lda) x Bk [Kb, N]; see k_prompt_down.
static void launch_down(hipStream_t st, const uint16_t* A, int M, int lda, int Ka, const bf16s* Bk, int Kb, int N,
                        float* Y) {
  const int mt = (M + kBM - 1) / kBM, nt = (N + kDnBN - 1) / kDnBN;
  POP_LAUNCH((k_prompt_down<POP_DOWN_NS, POP_PROMPT_GR>), dim3(mt * nt), dim3(kGuThreads), 0, st, A, M, lda, Ka, Bk, Kb, N, Y, mt,
             nt);
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
      launch_gateup(st, imp ? (mt >= 4 ? 4 : mt >= 2 ? 2 : 1) : 0, Xc, M, (int)d, (const bf16s*)Wg,
                    (const bf16s*)Wu, (int)d_ff, (uint16_t*)ws, ldz, s2, I);
      launch_down(st, (const uint16_t*)ws, M, ldz, ldz, (const bf16s*)WdT, (int)d_ff, (int)d, Yc);
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
      launch_down(st, (const uint16_t*)A + (int64_t)m0 * lda, Mc, lda, K, (const bf16s*)Bk, K, N, Yc);
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
