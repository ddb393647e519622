// fp32 GEMM through the fp16 matrix cores: operand preparation.
//
// The pages run fp32 GEMMs faster than the fp32 units allow by rounding the
// inputs to a narrower format ("SGEMM CUDA代码学习" 第5步, TF32 with WMMA), which
// loses accuracy.  This path keeps fp32 accuracy by splitting every input
// into two fp16 terms, the split-with-residual scheme of Markidis et al.
// (2018, "NVIDIA Tensor Core Programmability, Performance & Precision") with
// power-of-two scaling against fp16's narrow range (as in Ootomo and Yokota,
// 2022, "Recovering single precision accuracy from Tensor Cores while
// surpassing the FP32 theoretical peak performance"):
//
//   row r of op(A) (column r of op(B)) is scaled by 2^e_r, with e_r chosen so
//   that its largest magnitude lands in [2^14, 2^15) (below fp16's maximum);
//   each scaled value v splits into hi = fp16(v) and lo = fp16(v - hi), where
//   v - hi is exact in fp32, so v = hi + lo up to 2^-22 |v|;
//   a*b ~ hi_a*hi_b + hi_a*lo_b + lo_a*hi_b (the dropped lo_a*lo_b is below
//   2^-22 |a*b|), accumulated in fp32 by the MFMAs.
//
// The three products are one fp16 GEMM over K' = 3 Kp (Kp = K rounded up to
// a multiple of 64, zero-padded): the kernels here write
//   A' (M x 3Kp, row-major) = [hi | hi | lo] of op(A)'s rows,
//   B' (N x 3Kp, row-major) = [hi | lo | hi] of op(B)'s columns,
// so A' B'^T is the TN problem the fp16 tiles run, and the epilogue undoes
// the scaling with an exact ldexp by -(e_m + e_n).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "split16.hpp"

namespace mg {

namespace {

constexpr int kThreads = 256;

// Scale exponent for a row whose largest magnitude is mx: mx * 2^e lies in
// [2^14, 2^15).  Zero or non-finite rows keep e = 0.
__device__ __forceinline__ int scale_exp(float mx) {
  if (!(mx > 0.0f) || !isfinite(mx)) return 0;
  int q;
  frexpf(mx, &q);  // mx = f * 2^q, f in [0.5, 1)
  return 15 - q;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Row r of a row-contiguous op(X) (R x K at X + r * ld): one workgroup per row.
__global__ void __launch_bounds__(kThreads) rowmax_direct(const float *X, int64_t ld, int K, int *exp_out) {
  __shared__ float part[kThreads / 64];
  const int r = blockIdx.x;
  const float *row = X + (int64_t)r * ld;
  float m = 0.0f;
  for (int k = threadIdx.x; k < K; k += kThreads) m = fmaxf(m, fabsf(row[k]));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = part[0];
    for (int w = 1; w < kThreads / 64; ++w) t = fmaxf(t, part[w]);
    exp_out[r] = scale_exp(t);
  }
}

// op(X) row r is column r of a stored K x R matrix (X + k * ld + r): thread
// per column, K cut into gridDim.y ranges whose maxima go to pm[y * R + r].
__global__ void __launch_bounds__(kThreads) colmax_partial(const float *X, int64_t ld, int R, int K,
                                                           int kchunk, float *pm) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= R) return;
  const int k0 = blockIdx.y * kchunk, k1 = min(K, k0 + kchunk);
  float m = 0.0f;
  for (int k = k0; k < k1; ++k) m = fmaxf(m, fabsf(X[(int64_t)k * ld + r]));
  pm[(int64_t)blockIdx.y * R + r] = m;
}

__global__ void __launch_bounds__(kThreads) colmax_final(const float *pm, int R, int parts, int *exp_out) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= R) return;
  float m = 0.0f;
  for (int s = 0; s < parts; ++s) m = fmaxf(m, pm[(int64_t)s * R + r]);
  exp_out[r] = scale_exp(m);
}

// Writes the three segments of element (r, k) of the split operand.
// pattern 0: [hi | hi | lo] (the A side); 1: [hi | lo | hi] (the B side).
__device__ __forceinline__ void put(uint16_t *out, int64_t row_off, int Kp, int k, float v, int pattern) {
  const _Float16 hi = (_Float16)v;
  const _Float16 lo = (_Float16)(v - (float)hi);
  const uint16_t h = __builtin_bit_cast(uint16_t, hi), l = __builtin_bit_cast(uint16_t, lo);
  uint16_t *o = out + row_off + k;
  o[0] = h;
  o[Kp] = pattern == 0 ? h : l;
  o[2 * Kp] = pattern == 0 ? l : h;
}

// Row-contiguous source: grid (R, ceil(Kp / kThreads)), thread per k.
__global__ void __launch_bounds__(kThreads) split_direct(const float *X, int64_t ld, int K, int Kp,
                                                         const int *exps, uint16_t *out, int pattern) {
  const int r = blockIdx.x;
  const int k = blockIdx.y * kThreads + threadIdx.x;
  if (k >= Kp) return;
  const float v = k < K ? ldexpf(X[(int64_t)r * ld + k], exps[r]) : 0.0f;
  put(out, (int64_t)r * 3 * Kp, Kp, k, v, pattern);
}

// Column source (stored K x R): 64 x 64 tiles through LDS so that both the
// reads (along r) and the writes (along k) are contiguous.  Grid
// (ceil(Kp / 64), ceil(R / 64)), 256 threads.
__global__ void __launch_bounds__(kThreads) split_transposed(const float *X, int64_t ld, int R, int K, int Kp,
                                                             const int *exps, uint16_t *out, int pattern) {
  __shared__ float tile[64][65];
  const int k0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // ty: 0..3
  for (int kk = ty; kk < 64; kk += 4) {
    const int k = k0 + kk, r = r0 + tx;
    tile[kk][tx] = (k < K && r < R) ? X[(int64_t)k * ld + r] : 0.0f;
  }
  __syncthreads();
  for (int rr = ty; rr < 64; rr += 4) {
    const int r = r0 + rr, k = k0 + tx;
    if (r < R && k < Kp) put(out, (int64_t)r * 3 * Kp, Kp, k, ldexpf(tile[tx][rr], exps[r]), pattern);
  }
}

}  // namespace

hipError_t split16_prepare(const Split16Plan &s, hipStream_t stream) {
  // exponents of op(A)'s rows and op(B)'s columns
  auto exps = [&](const float *X, int64_t ld, int R, bool contiguous, int *exp_out) {
    if (contiguous) {
      hipLaunchKernelGGL(rowmax_direct, dim3(R), dim3(kThreads), 0, stream, X, ld, s.K, exp_out);
    } else {
      const int kchunk = (s.K + s.parts - 1) / s.parts;
      hipLaunchKernelGGL(colmax_partial, dim3((R + kThreads - 1) / kThreads, s.parts), dim3(kThreads), 0,
                         stream, X, ld, R, s.K, kchunk, s.pmax);
      hipLaunchKernelGGL(colmax_final, dim3((R + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                         s.pmax, R, s.parts, exp_out);
    }
  };
  auto split = [&](const float *X, int64_t ld, int R, bool contiguous, const int *e, uint16_t *out,
                   int pattern) {
    if (contiguous)
      hipLaunchKernelGGL(split_direct, dim3(R, (s.Kp + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                         X, ld, s.K, s.Kp, e, out, pattern);
    else
      hipLaunchKernelGGL(split_transposed, dim3((s.Kp + 63) / 64, (R + 63) / 64), dim3(kThreads), 0, stream,
                         X, ld, R, s.K, s.Kp, e, out, pattern);
  };
  // op(A) rows are contiguous when A is stored M x K; op(B) columns when B is
  // stored N x K.
  exps(s.A, s.lda, s.M, s.a_rows_contiguous, s.row_exp);
  exps(s.B, s.ldb, s.N, s.b_cols_contiguous, s.col_exp);
  split(s.A, s.lda, s.M, s.a_rows_contiguous, s.row_exp, s.Ap, 0);
  split(s.B, s.ldb, s.N, s.b_cols_contiguous, s.col_exp, s.Bp, 1);
  return hipGetLastError();
}

}  // namespace mg
