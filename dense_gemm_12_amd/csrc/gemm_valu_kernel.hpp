// fp32 SGEMM on the vector ALUs: the alternative that the f32 MFMA tiles are
// weighed against.  "SGEMM CUDA代码学习" steps 2-4 and the worklog's kernels
// 4-5 build the CUDA-core SGEMM as a register micro-tile per thread fed from
// shared memory; here each lane owns an 8 x 8 tile of C and runs plain
// v_fmac_f32 (packed fp32 ops are excluded from every build).  MI355X's fp32
// vector peak (157.3 TFLOP/s) equals its f32 MFMA peak, so the comparison is
// one of how much of that peak each path keeps.
//
// Staging reuses the direct-to-LDS operand layouts of the MFMA tiles
// (gemm_dma_kernel.hpp): a k-contiguous operand as [row][k] with permuted
// 16-byte chunks, a k-major one as [k][row].  Lane (tr, tc) of the 16 x 16
// grid owns rows 4 tr + 64 h + e and columns 4 tc + 64 h + e (h = 0, 1;
// e = 0..3), so the 16 lanes of a k-major read cover one contiguous 256-byte
// span (no bank conflicts) and each lane stores 4 consecutive columns.  Per
// group of 4 k values a lane reads its 8 rows of op(A) and 8 columns of op(B)
// with 16-byte LDS reads (8 per operand in either layout) and runs 256 FMAs.
// Two LDS stages: the DMA for slice kt+1 is in flight while slice kt is
// computed.
#pragma once
#include "epilogue.hpp"
#include "gemm_dma_kernel.hpp"

namespace mg {

template <int BM_, int BN_, int BK_, bool A_KC, bool B_KC>
struct ValuTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int NW = 4, NT = 256, TM = 8, TN = 8;
  static_assert(BM == 16 * TM && BN == 16 * TN, "16 x 16 lanes of 8 x 8 micro-tiles");
  static_assert(BK % 4 == 0, "k in groups of four");
  using OA = DmaOperand<BM, BK, A_KC, NW, 4>;
  using OB = DmaOperand<BN, BK, B_KC, NW, 4>;
  static constexpr int STAGE_BYTES = OA::BYTES + OB::BYTES;
  static constexpr int LOADS = OA::INST + OB::INST;

  // Row i (0..7) of a lane whose group index is t: 4 t + 64 (i / 4) + i % 4.
  static __device__ __forceinline__ int own(int t, int i) { return 4 * t + 64 * (i >> 2) + (i & 3); }

  // Four k values (k4*4 .. +3) of the lane's 8 operand rows: v[r][kk].  KC:
  // one 16-byte read per row; k-major: two per k.
  template <class O, bool KC>
  static __device__ __forceinline__ void read8x4(const char *st, int t, int k4, float (&v)[8][4]) {
    if constexpr (KC) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int row = own(t, r);
        const f32x4 x = *reinterpret_cast<const f32x4 *>(st + row * O::ROWB + ((k4 ^ O::swz(row)) * 16));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) v[r][kk] = x[kk];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const char *p = st + (k4 * 4 + kk) * O::ROWB + 16 * t;
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 x1 = *reinterpret_cast<const f32x4 *>(p + 256);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r][kk] = x0[r];
          v[r + 4][kk] = x1[r];
        }
      }
    }
  }

  static __device__ __forceinline__ void run(const GemmParams &p) {
    __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tr = tid >> 4, tc = tid & 15;  // this lane's rows own(tr, i), columns own(tc, j)

    int tm, tn, kb, K;
    work_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, p.K, p.k_chunk, tm, tn, kb, K);
    const int m0 = tm * BM, n0 = tn * BN;
    const char *Ab = static_cast<const char *>(p.A) +
                     (A_KC ? (int64_t)m0 * p.lda + kb : (int64_t)kb * p.lda + m0) * 4;
    const char *Bb = static_cast<const char *>(p.B) +
                     (B_KC ? (int64_t)n0 * p.ldb + kb : (int64_t)kb * p.ldb + n0) * 4;
    const int64_t a_step = (A_KC ? BK : (int64_t)BK * p.lda) * 4;
    const int64_t b_step = (B_KC ? BK : (int64_t)BK * p.ldb) * 4;
    const uint32_t lda_b = (uint32_t)(p.lda * 4), ldb_b = (uint32_t)(p.ldb * 4);
    const int rva = p.M - m0, rvb = p.N - n0;
    const int nk = (K + BK - 1) / BK;

    auto issue = [&](int kt) {
      char *st = lds + (kt & 1) * STAGE_BYTES;
      const int kv = K - kt * BK;
#pragma unroll
      for (int u = 0; u < OA::INST; ++u)
        OA::dma(make_rsrc(Ab + kt * a_step), lda_b, rva, kv, st, wave, lane, u);
#pragma unroll
      for (int u = 0; u < OB::INST; ++u)
        OB::dma(make_rsrc(Bb + kt * b_step), ldb_b, rvb, kv, st + OA::BYTES, wave, lane, u);
    };

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    if (nk > 0) issue(0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) issue(kt + 1);  // into the buffer every wave finished before the last barrier
      const char *st = lds + (kt & 1) * STAGE_BYTES;
#pragma unroll
      for (int k4 = 0; k4 < BK / 4; ++k4) {
        float a[8][4], b[8][4];
        read8x4<OA, A_KC>(st, tr, k4, a);
        read8x4<OB, B_KC>(st + OA::BYTES, tc, k4, b);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i][kk], b[j][kk], acc[i][j]);
      }
      wait_vmcnt<0>();  // slice kt+1 has landed
      __syncthreads();  // and every wave is done with slice kt
    }

    // epilogue: rows m0 + own(tr, i), columns n0 + own(tc, 4h) .. +3
    const bool split = p.splits > 1;
    const GemmParams q = split ? partial_params(p, kb) : p;
    const bool use_beta = q.beta != 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + own(tr, i);
      if (m >= q.M) continue;
      float *crow = static_cast<float *>(q.C) + (int64_t)m * q.ldc;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + own(tc, 4 * h);
        if (n >= q.N) continue;
        float x[4] = {acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]};
        if (!split && q.row_exp != nullptr) GemmEpilogue<float, 1, 1>::unscale(q, m, n, x);
        GemmEpilogue<float, 1, 1>::store4(q, crow, n, x, use_beta);
      }
    }
  }
};

template <class Tile>
__global__ void __launch_bounds__(Tile::NT) gemm_valu_kernel(GemmParams p) {
  Tile::run(p);
}

}  // namespace mg
