// Operand preparation for the fp32 GEMM through fp16 matrix cores (see
// split16.hip for the method).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

struct Split16Plan {
  const float *A, *B;     // the caller's fp32 operands (stored matrices)
  int64_t lda, ldb;
  int M, N, K;
  int Kp;                 // K rounded up to a multiple of 64 (segment width)
  bool a_rows_contiguous; // A stored M x K (op = N)
  bool b_cols_contiguous; // B stored N x K (op = T)
  int parts;              // K ranges for the strided-max pass
  // workspace sections
  uint16_t *Ap;           // M x 3Kp fp16: [hi | hi | lo]
  uint16_t *Bp;           // N x 3Kp fp16: [hi | lo | hi]
  int *row_exp;           // M
  int *col_exp;           // N
  float *pmax;            // parts x max(M, N) partial maxima
};

// Launches the exponent and split kernels on `stream`.
hipError_t split16_prepare(const Split16Plan &s, hipStream_t stream);

}  // namespace mg
