// f16-input GEMM configurations whose accumulators fit in VGPRs (v_mfma_f32_16x16x32_f16,
// fp32 accumulate; output f16 or fp32).  This file is compiled with MFMA
// operands kept in VGPRs (build.py explains why); the 256 x 256 tiles of four
// waves, which need AGPRs, live in kernels_f16.hip.
#include "kernels_inst.hpp"

namespace mg {

const KernelEntry *entries_f16_vgpr(int *n) {
  static const KernelEntry table[] = {
      make_dma_entry<_Float16, _Float16, 256, 256, 64, 2, 2, 4>("dma_f16_256x256x64_s2_w2x4"),
      make_dma_entry<_Float16, _Float16, 256, 256, 32, 4, 2, 4>("dma_f16_256x256x32_s4_w2x4"),
      make_dma_entry<_Float16, _Float16, 256, 128, 64, 2, 2, 2>("dma_f16_256x128x64_s2_w2x2"),
      make_dma_entry<_Float16, _Float16, 256, 128, 32, 4, 2, 2>("dma_f16_256x128x32_s4_w2x2"),
      make_dma_entry<_Float16, _Float16, 128, 128, 64, 3, 2, 2>("dma_f16_128x128x64_s3_w2x2"),
      // eight waves (64 x 32 each, two per SIMD): one covers the other's barrier
      make_dma_entry<_Float16, _Float16, 128, 128, 64, 3, 2, 4>("dma_f16_128x128x64_s3_w2x4"),
      make_dma_entry<_Float16, _Float16, 128, 128, 64, 4, 2, 4>("dma_f16_128x128x64_s4_w2x4"),
      make_entry<_Float16, _Float16, 256, 128, 64, 2, 2, true, true>("mfma_f16_256x128x64_w2x2"),
      make_entry<_Float16, _Float16, 128, 256, 64, 2, 2, true, true>("mfma_f16_128x256x64_w2x2"),
      make_entry<_Float16, _Float16, 128, 128, 64, 2, 2, true, true>("mfma_f16_128x128x64_w2x2"),
      make_entry<_Float16, _Float16, 64, 64, 64, 2, 2, true, true>("mfma_f16_64x64x64_w2x2"),
      make_entry<_Float16, _Float16, 128, 128, 64, 2, 2, false, true>("elemA_f16_128x128x64_w2x2"),
      make_entry<_Float16, _Float16, 128, 128, 64, 2, 2, true, false>("elemB_f16_128x128x64_w2x2"),
      make_entry<_Float16, _Float16, 128, 128, 64, 2, 2, false, false>("elemAB_f16_128x128x64_w2x2"),
      make_dma_entry<_Float16, _Float16, 256, 256, 32, 4, 2, 4, true>("dma_f16_256x256x32_s4_w2x4_pp"),
      make_dma_entry<_Float16, _Float16, 256, 256, 32, 4, 4, 2, true>("dma_f16_256x256x32_s4_w4x2_pp"),
      make_ws_entry<_Float16, _Float16, 256, 128, 32, 6, 2, 2>("ws_f16_256x128x32_s6_w2x2"),
      make_ws_entry<_Float16, _Float16, 128, 256, 32, 6, 2, 2>("ws_f16_128x256x32_s6_w2x2"),
      make_ws_entry<_Float16, _Float16, 256, 128, 32, 4, 2, 2>("ws_f16_256x128x32_s4_w2x2"),
      make_dma_entry<_Float16, _Float16, 256, 256, 64, 2, 2, 4, false, true>("dma_f16_256x256x64_s2_w2x4_sk"),
      // few-row problems (split over K): A stored M x K only; four waves, or eight (two per SIMD)
      make_dma_entry<_Float16, _Float16, 64, 128, 64, 3, 2, 2>("dma_f16_64x128x64_s3_w2x2"),
      make_dma_entry<_Float16, _Float16, 64, 128, 64, 4, 2, 4>("dma_f16_64x128x64_s4_w2x4"),
  };
  *n = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace mg
