// The prompt pass's matrix-core GEMM, shared with the decoder layer's prompt
// pass (host side, defined in prompt_ffn.hip).
#pragma once
#include <stdint.h>

#include "../../include/pop.h"

namespace pop {

// Y [M, N] (fp32, row-major) = A [M, K] * Bk [K, N], A and Bk in dt, Bk
// K-major (row k holds the N outputs' weights of input k).  A's row pitch is
// lda elements.  bf16: the down-projection kernel of the prompt FFN
// (v_mfma_f32_16x16x32_bf16), which needs K % 64 == 0 (or zeros in A past K up
// to the next multiple of 64), N % 8 == 0 and M >= 1; fp32: LDS-tiled FMA.
// ksplit > 1 (bf16, M <= 4096; otherwise one slice): the reduction is split
// into ceil(K / kslice) slices of kslice = K / ksplit rounded up to 64 rows,
// and Y holds one partial product per slice, [slices][M][N], for the caller
// to sum.  Returns the number of slices written (1: Y is the whole product);
// at most gemm_kslices(K, ksplit).  Enqueued on `stream` (a hipStream_t); no
// checks.
int launch_gemm_kmajor(void* stream, const void* A, int M, int lda, const void* Bk, int K, int N, pop_dtype dt,
                       float* Y, int ksplit = 1);

// The number of slices a split over (K, ksplit) makes (a bound for sizing Y).
inline int gemm_kslices(int K, int ksplit) {
  if (ksplit <= 1) return 1;
  const int kslice = (K / ksplit + 63) / 64 * 64;
  return (K + kslice - 1) / kslice;
}

}  // namespace pop
