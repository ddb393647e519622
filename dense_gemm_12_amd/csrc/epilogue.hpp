// Fused epilogue shared by the GEMM kernels: C = alpha * acc + beta * C in
// fp32, one rounding (nearest-even) to the output type, every row and column
// tail masked.  beta == 0 never reads C.  ("CUDA GEMM：从基础写法到工程优化" section 1
// and the worklog's Kernel 1 apply alpha/beta per output element; here the
// update is fused into the tile's register epilogue.)
#pragma once
#include "gemm_params.hpp"
#include "gfx950_prims.hpp"

namespace mg {

// Accumulator layout: acc[i][j] is the 16x16 block (i, j) of the wave's
// sub-tile; lane l holds 4 consecutive columns n = nw + j*16 + 4*(l/16) .. +3
// of row m = mw + i*16 + l%16.
template <typename TO, int MI, int NJ>
struct GemmEpilogue {
  // C[m][n..n+3] for m = mw + i*16 + lane%16, n = nw + j*16 + 4*(lane/16).
  static __device__ __forceinline__ void store(const GemmParams &p, const f32x4 (&acc)[MI][NJ],
                                               int mw, int nw, int lane) {
    TO *C = static_cast<TO *>(p.C);
    const float alpha = p.alpha, beta = p.beta;
    const bool use_beta = beta != 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = mw + i * 16 + (lane & 15);
      if (m >= p.M) continue;
      TO *crow = C + (int64_t)m * p.ldc;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = nw + j * 16 + (lane >> 4) * 4;
        if (n >= p.N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][e];
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
              float x = v[e];
              if (use_beta) x = fmaf(beta, to_f32(crow[n + e]), x);
              crow[n + e] = from_f32<TO>(x);
            }
          }
        }
      }
    }
  }
};

}  // namespace mg
