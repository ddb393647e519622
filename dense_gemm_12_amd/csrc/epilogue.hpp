// Fused epilogue shared by the GEMM kernels: C = alpha * acc + beta * C in
// fp32, one rounding (nearest-even) to the output type, every row and column
// tail masked.  beta == 0 never reads C.  ("CUDA GEMM：从基础写法到工程优化" section 1
// and the worklog's Kernel 1 apply alpha/beta per output element; here the
// update is fused into the tile's register epilogue.)
#pragma once
#include <type_traits>

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
template <typename TO, int MI, int NJ, bool RQ = false, bool CQ = false, bool WIDE = true>
struct GemmEpilogue {
  static_assert(!RQ || MI % 4 == 0, "row quads need whole quads");
  static_assert(!CQ || NJ % 4 == 0, "column quads need whole quads");

  // Four C values as stored: 16 bytes of fp32, 8 bytes of a 16-bit type.
  using Raw4 = typename std::conditional<sizeof(TO) == 4, f32x4, u32x2>::type;

  // Whether C[m][n .. n+3] is one vector access.
  static __device__ __forceinline__ bool vec4(const GemmParams &p, int n) { return p.c_vec && n + 3 < p.N; }
  static __device__ __forceinline__ Raw4 load4(const TO *crow, int n) {
    return *reinterpret_cast<const Raw4 *>(crow + n);
  }

  // C[m][n .. n+3] = alpha * x + beta * c for a vector access (vec4), with c
  // the four values load4 read before (used only with use_beta).
  static __device__ __forceinline__ void store4v(const GemmParams &p, TO *crow, int n, const float (&x)[4],
                                                 bool use_beta, const Raw4 &c) {
    const float alpha = p.alpha, beta = p.beta;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = alpha * x[e];
    if constexpr (sizeof(TO) == 4) {
      if (use_beta) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(beta, c[e], v[e]);
      }
      *reinterpret_cast<f32x4 *>(crow + n) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
      if (use_beta) {
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
      *reinterpret_cast<u32x2 *>(crow + n) = o;
    }
  }

  // C[m][n .. n+3] = alpha * x + beta * C, masked at the column tail.
  static __device__ __forceinline__ void store4(const GemmParams &p, TO *crow, int n, const float (&x)[4],
                                                bool use_beta) {
    if (vec4(p, n)) {
      store4v(p, crow, n, x, use_beta, use_beta ? load4(crow, n) : Raw4{});
    } else {
      const float alpha = p.alpha, beta = p.beta;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = alpha * x[e];
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

  // Column quads store badly as they are: component v of block 4q + c is
  // column 16g + 4v + c of the quad (g = lane / 16), so one store instruction
  // would cover each row in four 16-byte pieces 64 bytes apart (measured: the
  // fp32 NN 256 x 256 tiles lost ~6 % to it).  A 4 x 4 transpose of (lane
  // group, component) with the lane-row swaps of gfx950 (v_permlane32_swap:
  // lane groups 2, 3 of the first operand <-> 0, 1 of the second;
  // v_permlane16_swap: groups 1, 3 of the first <-> 0, 2 of the second; each
  // lane keeps its position within its group) turns component v of lane
  // group g into column 16v + 4g + c, so that every store covers 64
  // contiguous bytes of a row.  A group and its partners hold the same rows,
  // so they are active together.
  static __device__ __forceinline__ void transpose_quad(f32x4 &b) {
    // (element values first: a bit cast of an ext-vector element lvalue reads element 0)
    const float f0 = b[0], f1 = b[1], f2 = b[2], f3 = b[3];
    uint32_t r0 = __builtin_bit_cast(uint32_t, f0), r1 = __builtin_bit_cast(uint32_t, f1);
    uint32_t r2 = __builtin_bit_cast(uint32_t, f2), r3 = __builtin_bit_cast(uint32_t, f3);
    auto s02 = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    b = f32x4{__builtin_bit_cast(float, (uint32_t)s01[0]), __builtin_bit_cast(float, (uint32_t)s01[1]),
              __builtin_bit_cast(float, (uint32_t)s23[0]), __builtin_bit_cast(float, (uint32_t)s23[1])};
  }

  // 16-bit C: lane group g holds columns 4g .. 4g + 3 of each 16-column
  // block, so a store covers 32 bytes of a row.  For a pair of blocks
  // (a = block 2jj, b = block 2jj + 1), v_permlane32_swap(a, b) then
  // v_permlane16_swap on the results leave lane group g with columns
  // 8g .. 8g + 7 of the 32-column pair (first four in a, last four in b),
  // so each lane stores 16 bytes and a store covers 64 contiguous bytes of a
  // row (measured: fp16 TN 4096^3 3 % faster).
  static __device__ __forceinline__ void transpose_pair(f32x4 &a, f32x4 &b) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float fa = a[c], fb = b[c];  // element values first (see transpose_quad)
      auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, fa), __builtin_bit_cast(uint32_t, fb),
                                                false, false);
      auto t = __builtin_amdgcn_permlane16_swap(s[0], s[1], false, false);
      a[c] = __builtin_bit_cast(float, (uint32_t)t[0]);
      b[c] = __builtin_bit_cast(float, (uint32_t)t[1]);
    }
  }

  // C[m][n .. n+7] = alpha * x + beta * C for 16-bit C: one 16-byte access
  // where the row allows it (c_vec >= 2), else two four-column stores.
  static __device__ __forceinline__ bool vec8(const GemmParams &p, int n) { return p.c_vec >= 2 && n + 7 < p.N; }
  static __device__ __forceinline__ u32x4 load8(const TO *crow, int n) {
    return *reinterpret_cast<const u32x4 *>(crow + n);
  }
  // The 16-byte access of store8 with c read before by load8.
  static __device__ __forceinline__ void store8v(const GemmParams &p, TO *crow, int n, const float (&x)[8],
                                                 bool use_beta, const u32x4 &c) {
    static_assert(sizeof(TO) == 2, "16-bit output");
    const float alpha = p.alpha, beta = p.beta;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = alpha * x[e];
    if (use_beta) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t bits = (uint16_t)(c[e >> 1] >> (16 * (e & 1)));
        v[e] = fmaf(beta, to_f32(__builtin_bit_cast(TO, bits)), v[e]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, from_f32<TO>(v[2 * d]));
      const uint32_t hi = __builtin_bit_cast(uint16_t, from_f32<TO>(v[2 * d + 1]));
      o[d] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4 *>(crow + n) = o;
  }
  static __device__ __forceinline__ void store8(const GemmParams &p, TO *crow, int n, const float (&x)[8],
                                                bool use_beta) {
    static_assert(sizeof(TO) == 2, "16-bit output");
    if (vec8(p, n)) {
      store8v(p, crow, n, x, use_beta, use_beta ? load8(crow, n) : u32x4{});
    } else {
      const float x0[4] = {x[0], x[1], x[2], x[3]}, x1[4] = {x[4], x[5], x[6], x[7]};
      store4(p, crow, n, x0, use_beta);
      store4(p, crow, n + 4, x1, use_beta);
    }
  }

  // Four-column stores are kept where registers are short: with WIDE =
  // false (the stream-K tiles: the pair transpose's registers, live across
  // their loop over work units, pushed the register allocator into reusing
  // an in-flight LDS read's destination) and for more than 32 accumulator
  // blocks per lane (the four-wave 256 x 256 tiles, which then spilled).
  static constexpr bool PAIRS = WIDE && !CQ && sizeof(TO) == 2 && NJ % 2 == 0 && MI * NJ <= 32;

  static __device__ __forceinline__ void store(const GemmParams &p, const f32x4 (&acc)[MI][NJ],
                                               int mw, int nw, int lane) {
    TO *C = static_cast<TO *>(p.C);
    const bool use_beta = p.beta != 0.0f;
    const bool scaled = p.row_exp != nullptr;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      f32x4 blk[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        blk[j] = acc[i][j];
        if constexpr (CQ) transpose_quad(blk[j]);  // before any lane leaves the loop
      }
      if constexpr (PAIRS) {
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj) transpose_pair(blk[2 * jj], blk[2 * jj + 1]);
      }
      const int m = RQ ? mw + 64 * (i >> 2) + 4 * r + (i & 3) : mw + i * 16 + r;
      if (m >= p.M) continue;
      TO *crow = C + (int64_t)m * p.ldc;
      // With beta != 0 every vector access of the row is loaded before the
      // first store: issued one by one after each store, the loads waited
      // out a memory round trip each (the bf16 NN 4096 x 11008 x 4096 tile's
      // fp32 C read took ~20 us a round that way).
      if constexpr (PAIRS) {
        u32x4 cin[NJ / 2] = {};
        if (use_beta) {
#pragma unroll
          for (int jj = 0; jj < NJ / 2; ++jj)
            if (vec8(p, nw + jj * 32 + g * 8)) cin[jj] = load8(crow, nw + jj * 32 + g * 8);
        }
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj) {
          const int n = nw + jj * 32 + g * 8;  // after transpose_pair
          if (n >= p.N) continue;
          float x[8] = {blk[2 * jj][0],     blk[2 * jj][1],     blk[2 * jj][2],     blk[2 * jj][3],
                        blk[2 * jj + 1][0], blk[2 * jj + 1][1], blk[2 * jj + 1][2], blk[2 * jj + 1][3]};
          if (scaled) {
            float x0[4] = {x[0], x[1], x[2], x[3]}, x1[4] = {x[4], x[5], x[6], x[7]};
            unscale(p, m, n, x0);
            unscale(p, m, n + 4, x1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[e] = x0[e];
              x[4 + e] = x1[e];
            }
          }
          if (vec8(p, n)) store8v(p, crow, n, x, use_beta, cin[jj]);
          else store8(p, crow, n, x, use_beta);
        }
      } else if constexpr (!CQ) {
        Raw4 cin[NJ] = {};
        if (use_beta) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            if (vec4(p, nw + j * 16 + g * 4)) cin[j] = load4(crow, nw + j * 16 + g * 4);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = nw + j * 16 + g * 4;
          if (n >= p.N) continue;
          float x[4] = {blk[j][0], blk[j][1], blk[j][2], blk[j][3]};
          if (scaled) unscale(p, m, n, x);
          if (vec4(p, n)) store4v(p, crow, n, x, use_beta, cin[j]);
          else store4(p, crow, n, x, use_beta);
        }
      } else {
        Raw4 cin[NJ] = {};
        if (use_beta) {
#pragma unroll
          for (int q = 0; q < NJ / 4; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (vec4(p, nw + 64 * q + 16 * v + 4 * g)) cin[4 * q + v] = load4(crow, nw + 64 * q + 16 * v + 4 * g);
        }
#pragma unroll
        for (int q = 0; q < NJ / 4; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = nw + 64 * q + 16 * v + 4 * g;  // after transpose_quad
            if (n >= p.N) continue;
            float x[4] = {blk[4 * q][v], blk[4 * q + 1][v], blk[4 * q + 2][v], blk[4 * q + 3][v]};
            if (scaled) unscale(p, m, n, x);
            if (vec4(p, n)) store4v(p, crow, n, x, use_beta, cin[4 * q + v]);
            else store4(p, crow, n, x, use_beta);
          }
      }
    }
  }
};

}  // namespace mg
