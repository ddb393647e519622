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

#include "gfx950_prims.hpp"
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
  float m[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  int k = k0;
  for (; k + 7 < k1; k += 8) {  // eight independent loads in flight
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], fabsf(X[(int64_t)(k + u) * ld + r]));
  }
  for (; k < k1; ++k) m[0] = fmaxf(m[0], fabsf(X[(int64_t)k * ld + r]));
#pragma unroll
  for (int u = 1; u < 8; ++u) m[0] = fmaxf(m[0], m[u]);
  pm[(int64_t)blockIdx.y * R + r] = m[0];
}

__global__ void __launch_bounds__(kThreads) colmax_final(const float *pm, int R, int parts, int *exp_out) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= R) return;
  float m[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  int s = 0;
  for (; s + 7 < parts; s += 8) {  // eight independent loads in flight
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], pm[(int64_t)(s + u) * R + r]);
  }
  for (; s < parts; ++s) m[0] = fmaxf(m[0], pm[(int64_t)s * R + r]);
#pragma unroll
  for (int u = 1; u < 8; ++u) m[0] = fmaxf(m[0], m[u]);
  exp_out[r] = scale_exp(m[0]);
}

// Writes the three segments of elements (r, k .. k+3) of the split operand
// (k a multiple of 4, so each segment store is one aligned 8-byte write).
// pattern 0: [hi | hi | lo] (the A side); 1: [hi | lo | hi] (the B side).
__device__ __forceinline__ void put4(uint16_t *out, int64_t row_off, int Kp, int k, const float (&v)[4],
                                     int pattern) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const _Float16 h0 = (_Float16)v[2 * d], h1 = (_Float16)v[2 * d + 1];
    const _Float16 l0 = (_Float16)(v[2 * d] - (float)h0), l1 = (_Float16)(v[2 * d + 1] - (float)h1);
    h[d] = __builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    l[d] = __builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  u32x2 *o = reinterpret_cast<u32x2 *>(out + row_off + k);
  const u32x2 hv = {h[0], h[1]}, lv = {l[0], l[1]};
  o[0] = hv;
  *reinterpret_cast<u32x2 *>(out + row_off + Kp + k) = pattern == 0 ? hv : lv;
  *reinterpret_cast<u32x2 *>(out + row_off + 2 * Kp + k) = pattern == 0 ? lv : hv;
}

// Row-contiguous source: grid (R, ceil(Kp / (4 kThreads))), four k per thread.
__global__ void __launch_bounds__(kThreads) split_direct(const float *X, int64_t ld, int K, int Kp,
                                                         const int *exps, uint16_t *out, int pattern) {
  const int r = blockIdx.x;
  const int k = (blockIdx.y * kThreads + threadIdx.x) * 4;
  if (k >= Kp) return;
  const float *row = X + (int64_t)r * ld;
  const int e = exps[r];
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = k + i < K ? ldexpf(row[k + i], e) : 0.0f;
  put4(out, (int64_t)r * 3 * Kp, Kp, k, v, pattern);
}

// Row-contiguous source with Kp <= kFusedMaxK: one workgroup per row reads
// the row once into registers (16-byte loads when vec), takes its largest
// magnitude, and writes the row's exponent and its split (the same values
// rowmax_direct and split_direct produce, from one read of the row).
constexpr int kFusedChunks = 16;  // four-element chunks per thread
constexpr int kFusedMaxK = kFusedChunks * 4 * kThreads;

__global__ void __launch_bounds__(kThreads) split_rows_fused(const float *X, int64_t ld, int K, int Kp, int vec,
                                                             int *exp_out, uint16_t *out, int pattern) {
  __shared__ float part[kThreads / 64];
  const int r = blockIdx.x;
  const float *row = X + (int64_t)r * ld;
  float v[kFusedChunks][4];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kFusedChunks; ++j) {
    const int k = (j * kThreads + threadIdx.x) * 4;
    if (vec && k + 3 < K) {
      const f32x4 x = *reinterpret_cast<const f32x4 *>(row + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[j][e] = x[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[j][e] = k + e < K ? row[k + e] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(v[j][e]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  float t = part[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) t = fmaxf(t, part[w]);
  const int ex = scale_exp(t);
  if (threadIdx.x == 0) exp_out[r] = ex;
#pragma unroll
  for (int j = 0; j < kFusedChunks; ++j) {
    const int k = (j * kThreads + threadIdx.x) * 4;
    if (k < Kp) {
      float w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = ldexpf(v[j][e], ex);
      put4(out, (int64_t)r * 3 * Kp, Kp, k, w4, pattern);
    }
  }
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
  // 16 threads per row, four k each; 16 rows per pass
  const int kq = (threadIdx.x & 15) * 4, rr0 = threadIdx.x >> 4;
  for (int rr = rr0; rr < 64; rr += 16) {
    const int r = r0 + rr, k = k0 + kq;
    if (r < R && k < Kp) {
      const int e = exps[r];
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ldexpf(tile[kq + i][rr], e);
      put4(out, (int64_t)r * 3 * Kp, Kp, k, v, pattern);
    }
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
      hipLaunchKernelGGL(split_direct, dim3(R, (s.Kp + 4 * kThreads - 1) / (4 * kThreads)), dim3(kThreads), 0,
                         stream,
                         X, ld, s.K, s.Kp, e, out, pattern);
    else
      hipLaunchKernelGGL(split_transposed, dim3((s.Kp + 63) / 64, (R + 63) / 64), dim3(kThreads), 0, stream,
                         X, ld, R, s.K, s.Kp, e, out, pattern);
  };
  // op(A) rows are contiguous when A is stored M x K; op(B) columns when B is
  // stored N x K.  Contiguous rows short enough for one pass take the fused
  // kernel.
  auto side = [&](const float *X, int64_t ld, int R, bool contiguous, int *e, uint16_t *out, int pattern) {
    if (contiguous && s.Kp <= kFusedMaxK) {
      const int vec = ((uintptr_t)X % 16 == 0 && ld % 4 == 0) ? 1 : 0;
      hipLaunchKernelGGL(split_rows_fused, dim3(R), dim3(kThreads), 0, stream, X, ld, s.K, s.Kp, vec, e, out,
                         pattern);
    } else {
      exps(X, ld, R, contiguous, e);
      split(X, ld, R, contiguous, e, out, pattern);
    }
  };
  side(s.A, s.lda, s.M, s.a_rows_contiguous, s.row_exp, s.Ap, 0);
  side(s.B, s.ldb, s.N, s.b_cols_contiguous, s.col_exp, s.Bp, 1);
  return hipGetLastError();
}

}  // namespace mg
