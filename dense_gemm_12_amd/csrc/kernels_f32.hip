// fp32 SGEMM configurations: v_mfma_f32_16x16x4_f32.  "dma_" tiles stage
// operands global -> LDS directly (every layout); "mfma_" tiles stage through
// registers; "elem" variants load element-wise where 16-byte loads are not
// legal.  "valu_" runs the same problem on v_fma_f32, for comparison (the
// planner's heuristic never picks it).
#include "kernels_inst.hpp"

namespace mg {

const KernelEntry *entries_f32(int *n) {
  static const KernelEntry table[] = {
      make_dma_entry<float, float, 256, 256, 32, 2, 2, 4>("dma_f32_256x256x32_s2_w2x4"),
      make_dma_entry<float, float, 256, 256, 16, 4, 2, 4>("dma_f32_256x256x16_s4_w2x4"),
      make_dma_entry<float, float, 256, 128, 32, 2, 2, 2>("dma_f32_256x128x32_s2_w2x2"),
      make_dma_entry<float, float, 128, 256, 32, 2, 2, 2>("dma_f32_128x256x32_s2_w2x2"),
      make_dma_entry<float, float, 128, 128, 32, 2, 2, 2>("dma_f32_128x128x32_s2_w2x2"),
      make_dma_entry<float, float, 128, 128, 16, 4, 2, 2>("dma_f32_128x128x16_s4_w2x2"),
      make_dma_entry<float, float, 128, 128, 16, 2, 2, 2>("dma_f32_128x128x16_s2_w2x2"),
      make_dma_entry<float, float, 128, 128, 16, 3, 2, 2>("dma_f32_128x128x16_s3_w2x2"),
      make_valu_entry<128, 128, 16>("valu_f32_128x128x16"),
      make_entry<float, float, 128, 128, 32, 2, 2, true, true>("mfma_f32_128x128x32_w2x2"),
      make_entry<float, float, 256, 128, 32, 2, 2, true, true>("mfma_f32_256x128x32_w2x2"),
      make_entry<float, float, 128, 256, 32, 2, 2, true, true>("mfma_f32_128x256x32_w2x2"),
      make_entry<float, float, 256, 256, 32, 2, 2, true, true>("mfma_f32_256x256x32_w2x2"),
      make_entry<float, float, 64, 64, 32, 2, 2, true, true>("mfma_f32_64x64x32_w2x2"),
      make_entry<float, float, 128, 128, 32, 2, 2, false, true>("elemA_f32_128x128x32_w2x2"),
      make_entry<float, float, 128, 128, 32, 2, 2, true, false>("elemB_f32_128x128x32_w2x2"),
      make_entry<float, float, 128, 128, 32, 2, 2, false, false>("elemAB_f32_128x128x32_w2x2"),
  };
  *n = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

template <typename TO>
static hipError_t launch_scale(const GemmParams &p, hipStream_t s) {
  const int64_t total = (int64_t)p.M * p.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(scale_c_kernel<TO>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename TO>
static hipError_t launch_reduce(const GemmParams &p, hipStream_t s) {
  const int64_t total = (int64_t)p.M * ((p.N + 3) / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(splitk_reduce_kernel<TO>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

LaunchFn reduce_launcher(int c_dtype) {
  switch (c_dtype) {
    case 0: return &launch_reduce<float>;
    case 1: return &launch_reduce<_Float16>;
    default: return &launch_reduce<__bf16>;
  }
}

hipError_t launch_pack(int es, const void *src, int64_t ld, int64_t rows, int64_t cols, void *dst,
                       int64_t pitch, hipStream_t s) {
  const int64_t total = rows * pitch;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) return hipSuccess;
  if (es == 4)
    hipLaunchKernelGGL(pack_rows_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, src, ld, rows, cols, dst,
                       pitch);
  else
    hipLaunchKernelGGL(pack_rows_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, src, ld, rows, cols, dst,
                       pitch);
  return hipGetLastError();
}

hipError_t launch_zero_ints(int *p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(zero_ints_kernel<0>, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

LaunchFn scale_launcher(int c_dtype) {
  switch (c_dtype) {
    case 0: return &launch_scale<float>;
    case 1: return &launch_scale<_Float16>;
    default: return &launch_scale<__bf16>;
  }
}

}  // namespace mg
