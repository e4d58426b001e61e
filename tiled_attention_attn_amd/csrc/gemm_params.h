// Kernel parameters of the in-kernel broadcast linear layer (ikbo_gemm.hip).
#ifndef ATTN_GEMM_PARAMS_H_
#define ATTN_GEMM_PARAMS_H_

#include <stdint.h>

namespace attn {

// One launch computes C[M, N] = A[M, K] B[N, K]^T, then adds bias[n] (if set)
// or, in the gathering form, row zrow[m] of Z[Mz, N]. A and B are bf16 with
// row strides lda / ldb elements; C is fp32 or bf16 with row stride N.
struct GemmParams {
  const void* a;
  const void* b;
  void* c;
  const float* bias;      // [N] or nullptr (non-gathering form only)
  const float* z;         // [Mz, N] fp32 (gathering form)
  const int32_t* zrow;    // [M] (gathering form)
  int M, N, K;
  int lda, ldb;           // elements
  int Mz;
  int tiles_n;            // ceil(N / tile)
  int tiles;              // ceil(M / tile) * tiles_n
};

}  // namespace attn

#endif  // ATTN_GEMM_PARAMS_H_
