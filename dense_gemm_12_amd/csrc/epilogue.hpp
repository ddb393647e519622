// Fused epilogue shared by the GEMM kernels: C = alpha * acc + beta * C in
// fp32, one rounding (nearest-even) to the output type, every row and column
// tail masked.  beta == 0 never reads C.  ("CUDA GEMM：从基础写法到工程优化" section 1
// and the worklog's Kernel 1 apply alpha/beta per output element; here the
// update is fused into the tile's register epilogue.)
#pragma once
#include "gemm_params.hpp"
#include "gfx950_prims.hpp"

namespace mg {

// Split-K: the epilogue of split s writes the raw fp32 sum (alpha = 1,
// beta = 0) to its slab of the workspace, rows of N floats.  kb is the
// split's first k.
__device__ __forceinline__ GemmParams partial_params(const GemmParams &p, int kb) {
  GemmParams q = p;
  const int s = kb / p.k_chunk;
  q.C = p.ws + (int64_t)s * p.M * p.N;
  q.ldc = p.N;
  q.alpha = 1.0f;
  q.beta = 0.0f;
  q.c_vec = (p.N % 4) == 0;
  q.row_exp = nullptr;  // partials are raw sums; the reduction unscales
  q.col_exp = nullptr;
  return q;
}

// Accumulator layout: acc[i][j] is the 16x16 block (i, j) of the wave's
// sub-tile and lane l holds its element (row position l%16, column positions
// 4*(l/16) + v, v = 0..3).  Positions map to C as follows.
//   rows, RQ = false: m = mw + 16i + l%16;
//   rows, RQ = true (row quads, see the fp32 k-major fragments):
//                     m = mw + 64(i/4) + 4(l%16) + i%4;
//   cols, CQ = false: n = nw + 16j + 4(l/16) + v, four consecutive columns;
//   cols, CQ = true:  n = nw + 64(j/4) + 16(l/16) + 4v + j%4, so the four
//                     blocks of a quad give each lane 16 consecutive columns.
template <typename TO, int MI, int NJ, bool RQ = false, bool CQ = false>
struct GemmEpilogue {
  static_assert(!RQ || MI % 4 == 0, "row quads need whole quads");
  static_assert(!CQ || NJ % 4 == 0, "column quads need whole quads");

  // C[m][n .. n+3] = alpha * x + beta * C, masked at the column tail.
  static __device__ __forceinline__ void store4(const GemmParams &p, TO *crow, int n, const float (&x)[4],
                                                bool use_beta) {
    const float alpha = p.alpha, beta = p.beta;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = alpha * x[e];
    if (p.c_vec && n + 3 < p.N) {
      if constexpr (sizeof(TO) == 4) {
        f32x4 *cp = reinterpret_cast<f32x4 *>(crow + n);
        if (use_beta) {
          const f32x4 c = *cp;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(beta, c[e], v[e]);
        }
        *cp = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        u32x2 *cp = reinterpret_cast<u32x2 *>(crow + n);
        if (use_beta) {
          const u32x2 c = *cp;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint16_t bits = (uint16_t)(c[e >> 1] >> (16 * (e & 1)));
            v[e] = fmaf(beta, to_f32(__builtin_bit_cast(TO, bits)), v[e]);
          }
        }
        u32x2 o;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t lo = __builtin_bit_cast(uint16_t, from_f32<TO>(v[2 * d]));
          const uint32_t hi = __builtin_bit_cast(uint16_t, from_f32<TO>(v[2 * d + 1]));
          o[d] = lo | (hi << 16);
        }
        *cp = o;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < p.N) {
          float y = v[e];
          if (use_beta) y = fmaf(beta, to_f32(crow[n + e]), y);
          crow[n + e] = from_f32<TO>(y);
        }
      }
    }
  }

  // x[e] *= 2^-(row_exp[m] + col_exp[n + e]) (exact unless the result leaves
  // fp32's range); masked tail columns read a valid exponent and are dropped.
  static __device__ __forceinline__ void unscale(const GemmParams &p, int m, int n, float (&x)[4]) {
    const int re = p.row_exp[m];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = ldexpf(x[e], -(re + p.col_exp[min(n + e, p.N - 1)]));
  }

  static __device__ __forceinline__ void store(const GemmParams &p, const f32x4 (&acc)[MI][NJ],
                                               int mw, int nw, int lane) {
    TO *C = static_cast<TO *>(p.C);
    const bool use_beta = p.beta != 0.0f;
    const bool scaled = p.row_exp != nullptr;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = RQ ? mw + 64 * (i >> 2) + 4 * r + (i & 3) : mw + i * 16 + r;
      if (m >= p.M) continue;
      TO *crow = C + (int64_t)m * p.ldc;
      if constexpr (!CQ) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = nw + j * 16 + g * 4;
          if (n >= p.N) continue;
          float x[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          if (scaled) unscale(p, m, n, x);
          store4(p, crow, n, x, use_beta);
        }
      } else {
#pragma unroll
        for (int q = 0; q < NJ / 4; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = nw + 64 * q + 16 * g + 4 * v;
            if (n >= p.N) continue;
            float x[4] = {acc[i][4 * q][v], acc[i][4 * q + 1][v], acc[i][4 * q + 2][v],
                          acc[i][4 * q + 3][v]};
            if (scaled) unscale(p, m, n, x);
            store4(p, crow, n, x, use_beta);
          }
      }
    }
  }
};

}  // namespace mg
