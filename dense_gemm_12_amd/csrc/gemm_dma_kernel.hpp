// 16-bit-input GEMM for operands whose k dimension is contiguous in memory
// (A stored M x K, B stored N x K: the "TN" layout of "HGEMM SMEM Swizzle
// 代码学习" and "Warp Specialization HGEMM" section 6), built around gfx950's
// global->LDS DMA:
//
//   * buffer_load_dwordx4 ... lds moves each 16-byte chunk from HBM straight
//     into LDS without passing through VGPRs, so no staging registers and no
//     ds_write instructions are spent on the copy;
//   * one DMA instruction writes 64 lanes x 16 bytes = 1 KiB of LDS at
//     consecutive addresses, so rows cannot be padded; bank conflicts on the
//     fragment reads are avoided instead by an XOR swizzle of the 16-byte
//     chunk index within each row (the idea "HGEMM SMEM Swizzle 代码学习"
//     applies to ldmatrix, re-derived here for CDNA4's LDS and wave64: the 16
//     rows one quarter-wave reads land in 16 distinct 16-byte bank groups of
//     a 256-byte window, and any 8 aligned rows in 8 distinct groups of a
//     128-byte window).  The DMA side applies the same permutation when it
//     picks which global chunk each lane fetches;
//   * STAGES slices ring through LDS: the loads for slice k+STAGES-1 are
//     issued right after the barrier that releases its buffer, so HBM latency
//     is covered by STAGES-1 slices of MFMA work ("SGEMM CUDA代码学习" step 5's
//     multistage pipeline, restated for vmcnt-counted DMA);
//   * each wave reads the fragments of the next k-step while the MFMAs of the
//     current one run (the two-level buffering the worklog's closing notes
//     describe).
// Tails: rows past M/N and k past K are fetched with an out-of-range buffer
// offset, which makes the DMA write zeros; slices beyond the last one are
// issued the same way so the vmcnt bookkeeping never changes.
#pragma once
#include "epilogue.hpp"
#include "gemm_params.hpp"
#include "gfx950_prims.hpp"

namespace mg {

typedef __attribute__((address_space(3))) void lds_void;

template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int r) {
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

template <typename TI, typename TO, int BM_, int BN_, int BK_, int STAGES_, int WAVES_M, int WAVES_N>
struct DmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int ROWB = BK * 2;              // LDS row bytes (16-bit elements)
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;          // rows per 1 KiB DMA block
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_INST = A_BYTES / 1024 / NW, B_INST = B_BYTES / 1024 / NW;
  static constexpr int LOADS_PER_SLICE = A_INST + B_INST;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int MI = WTM / 16, NJ = WTN / 16;
  static constexpr int KSTEPS = BK / 32;           // 16x16x32 MFMA k-steps per slice
  static_assert(CPR == 4 || CPR == 8, "BK must be 32 or 64");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole DMA blocks");
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LOADS_PER_SLICE * (STAGES - 1) < 64, "vmcnt range");

  // Issue the DMA for one operand slice.  base: byte address of stored
  // element (r0, k0); ldb: row pitch in bytes; rv/kv: rows and k left.
  template <int INST>
  static __device__ __forceinline__ void dma(const char *base, uint32_t ldb, int rv, int kv,
                                             char *lds, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
    const int slot = lane % CPR;
#pragma unroll
    for (int i = 0; i < INST; ++i) {
      const int blk = wave * INST + i;
      const int row = blk * RPB + lane / CPR;
      const int c = slot ^ chunk_swizzle<CPR>(row);
      const bool ok = row < rv && c * 8 < kv;
      const uint32_t off = ok ? row * ldb + c * 16 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds + blk * 1024), 16, off, 0, 0, 0);
    }
  }

  static __device__ __forceinline__ void run(const GemmParams &p) {
    __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    tile_coords(remap_xcd(blockIdx.x, p.tiles_m * p.tiles_n), p.tiles_m, p.tiles_n, p.group_m, tm,
                tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const char *Ab = static_cast<const char *>(p.A) + (int64_t)m0 * p.lda * 2;
    const char *Bb = static_cast<const char *>(p.B) + (int64_t)n0 * p.ldb * 2;
    const uint32_t lda_b = (uint32_t)(p.lda * 2), ldb_b = (uint32_t)(p.ldb * 2);
    const int rva = p.M - m0, rvb = p.N - n0;
    const int nk = (p.K + BK - 1) / BK;

    auto issue = [&](int kt) {
      char *st = lds + (kt % STAGES) * STAGE_BYTES;
      const int kv = p.K - kt * BK;
      dma<A_INST>(Ab + (int64_t)kt * BK * 2, lda_b, rva, kv, st, wave, lane);
      dma<B_INST>(Bb + (int64_t)kt * BK * 2, ldb_b, rvb, kv, st + A_BYTES, wave, lane);
    };

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Per-lane fragment offsets: row (lane % 16) of each 16-row block, chunk
    // (ks*4 + lane/16) un-swizzled by the row's pattern (which only depends
    // on the row modulo 16).
    const int lrow = lane & 15;
    const int sw = chunk_swizzle<CPR>(lrow);
    int coff[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) coff[ks] = (((ks * 4 + (lane >> 4)) ^ sw) * 16);
    const int a_row0 = (wm * WTM + lrow) * ROWB;
    const int b_row0 = A_BYTES + (wn * WTN + lrow) * ROWB;

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s);

    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<LOADS_PER_SLICE * (STAGES - 2)>();
      __syncthreads();
      issue(kt + STAGES - 1);
      const char *st = lds + (kt % STAGES) * STAGE_BYTES;
      u32x4 fa[2][MI], fb[2][NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        fa[0][i] = *reinterpret_cast<const u32x4 *>(st + a_row0 + i * 16 * ROWB + coff[0]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[0][j] = *reinterpret_cast<const u32x4 *>(st + b_row0 + j * 16 * ROWB + coff[0]);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        if (ks + 1 < KSTEPS) {
#pragma unroll
          for (int i = 0; i < MI; ++i)
            fa[nxt][i] = *reinterpret_cast<const u32x4 *>(st + a_row0 + i * 16 * ROWB + coff[ks + 1]);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            fb[nxt][j] = *reinterpret_cast<const u32x4 *>(st + b_row0 + j * 16 * ROWB + coff[ks + 1]);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) Mfma<TI>::step(acc[i][j], fb[cur][j], fa[cur][i]);
      }
    }

    GemmEpilogue<TO, MI, NJ>::store(p, acc, m0 + wm * WTM, n0 + wn * WTN, lane);
  }
};

template <class Tile>
__global__ void __launch_bounds__(Tile::NT) gemm_dma_kernel(GemmParams p) {
  Tile::run(p);
}

}  // namespace mg
