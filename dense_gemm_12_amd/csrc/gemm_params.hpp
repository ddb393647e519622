// Launch parameters shared by the host planner and the kernels, and the
// registry of compiled kernel configurations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

struct GemmParams {
  const void *A;
  const void *B;
  void *C;
  int64_t lda, ldb, ldc;  // elements
  int M, N, K;
  float alpha, beta;
  int tiles_m, tiles_n;   // grid = tiles_m * tiles_n workgroups
  int group_m;            // tile-rows per raster group
  int c_vec;              // C rows allow 16-byte (fp32) / 8-byte (16-bit) access; 2: 16-byte 16-bit too
  // Split-K.  splits == 1: one workgroup per tile covers all of K and the
  // epilogue writes C.  splits > 1: the grid is tiles * splits, split s
  // covers k in [s * k_chunk, min(K, (s + 1) * k_chunk)) and writes its fp32
  // partial tile to ws + s * M * N (row pitch N); a reduction kernel then
  // sums the partials in split order and applies alpha and beta.
  int splits;
  int k_chunk;            // multiple of every tile's BK
  float *ws;
  // Power-of-two unscaling of the product (fp32 through split fp16 inputs):
  // when row_exp is non-null, element (m, n) of the product is multiplied by
  // 2^-(row_exp[m] + col_exp[n]) before alpha and beta are applied.
  const int *row_exp;
  const int *col_exp;
  // Stream-K (configurations marked sk): sk_dp_tiles + sk_grid workgroups;
  // the first sk_dp_tiles each take one whole tile, the last sk_grid share
  // the slice iterations of the other tiles (sk_ipt per tile) in equal
  // contiguous ranges; partial tiles go to ws (2 * sk_grid slots of BM * BN
  // floats) and sk_cnt holds one zero-initialised arrival counter per tile.
  int sk_grid;
  int sk_ipt;
  int sk_dp_tiles;  // leading tiles dealt whole (a multiple of sk_grid); the rest is split
  int *sk_cnt;
};

typedef hipError_t (*LaunchFn)(const GemmParams &, hipStream_t);

// One compiled tile configuration; fn[c_is_f32][a_kc][b_kc] covers the
// output type and the four storage layouts (a_kc: A stored M x K; b_kc: B
// stored N x K); a null entry means the layout is not supported by this
// configuration.  a_vec / b_vec tell whether the variant needs
// 16-byte-loadable operands.  kind: 0 = register-staged loads, 1 = direct
// global->LDS loads.
typedef int (*OccupancyFn)();  // workgroups per CU of the kernel, -1 when it cannot be asked

struct KernelEntry {
  const char *name;
  int bm, bn, bk;
  bool a_vec, b_vec;
  int kind;
  LaunchFn fn[2][2][2];
  int threads;          // workgroup size
  int lds_bytes;        // static LDS per workgroup
  OccupancyFn occupancy;  // asked of the HIP runtime for one representative layout
  bool sk;              // stream-K schedule: needs a workspace (gemm_ex), never picked by the cost model
};

const KernelEntry *entries_f32(int *n);
const KernelEntry *entries_f16(int *n);
const KernelEntry *entries_bf16(int *n);
const KernelEntry *entries_f16_vgpr(int *n);   // the configurations compiled with VGPR-form MFMAs
const KernelEntry *entries_bf16_vgpr(int *n);

LaunchFn scale_launcher(int c_dtype);   // 0 = f32, 1 = f16, 2 = bf16
LaunchFn reduce_launcher(int c_dtype);  // split-K partial sums -> C, same codes
// Zeroes n ints (stream-K arrival counters) on the stream.
hipError_t launch_zero_ints(int *p, int n, hipStream_t s);
// Copies a rows x cols operand (es-byte elements) into a zero-padded buffer
// with a 16-byte-multiple row pitch.
hipError_t launch_pack(int es, const void *src, int64_t ld, int64_t rows, int64_t cols, void *dst,
                       int64_t pitch, hipStream_t s);

}  // namespace mg
