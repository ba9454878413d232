// The prompt pass's matrix-core GEMM, shared with the decoder layer's prompt
// pass (host side, defined in prompt_ffn.hip).
#pragma once
#include <stdint.h>

#include "../../include/pop.h"

namespace pop {

// Y [M, N] (fp32, row-major) = A [M, K] * Bk [K, N], A and Bk in dt, Bk
// K-major (row k holds the N outputs' weights of input k).  A's row pitch is
// lda elements.  bf16: the down-projection kernel of the prompt FFN
// (v_mfma_f32_16x16x32_bf16), which needs K % 8 == 0, N % 8 == 0 and M >= 1;
// fp32: LDS-tiled FMA.
// Enqueued on `stream` (a hipStream_t); no checks.
void launch_gemm_kmajor(void* stream, const void* A, int M, int lda, const void* Bk, int K, int N, pop_dtype dt,
                        float* Y);

}  // namespace pop
