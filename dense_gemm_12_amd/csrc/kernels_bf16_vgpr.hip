// bf16-input GEMM configurations whose accumulators fit in VGPRs (v_mfma_f32_16x16x32_bf16,
// fp32 accumulate; output bf16 or fp32).  This file is compiled with MFMA
// operands kept in VGPRs (build.py explains why); the 256 x 256 tiles of four
// waves, which need AGPRs, live in kernels_bf16.hip.
#include "kernels_inst.hpp"

namespace mg {

const KernelEntry *entries_bf16_vgpr(int *n) {
  static const KernelEntry table[] = {
      make_dma_entry<__bf16, __bf16, 256, 256, 64, 2, 2, 4>("dma_bf16_256x256x64_s2_w2x4"),
      make_dma_entry<__bf16, __bf16, 256, 256, 32, 4, 2, 4>("dma_bf16_256x256x32_s4_w2x4"),
      make_dma_entry<__bf16, __bf16, 256, 128, 64, 2, 2, 2>("dma_bf16_256x128x64_s2_w2x2"),
      make_dma_entry<__bf16, __bf16, 256, 128, 32, 4, 2, 2>("dma_bf16_256x128x32_s4_w2x2"),
      make_dma_entry<__bf16, __bf16, 128, 128, 64, 3, 2, 2>("dma_bf16_128x128x64_s3_w2x2"),
      // eight waves (64 x 32 each, two per SIMD): one covers the other's barrier
      make_dma_entry<__bf16, __bf16, 128, 128, 64, 3, 2, 4>("dma_bf16_128x128x64_s3_w2x4"),
      make_dma_entry<__bf16, __bf16, 128, 128, 64, 4, 2, 4>("dma_bf16_128x128x64_s4_w2x4"),
      make_entry<__bf16, __bf16, 256, 128, 64, 2, 2, true, true>("mfma_bf16_256x128x64_w2x2"),
      make_entry<__bf16, __bf16, 128, 256, 64, 2, 2, true, true>("mfma_bf16_128x256x64_w2x2"),
      make_entry<__bf16, __bf16, 128, 128, 64, 2, 2, true, true>("mfma_bf16_128x128x64_w2x2"),
      make_entry<__bf16, __bf16, 64, 64, 64, 2, 2, true, true>("mfma_bf16_64x64x64_w2x2"),
      make_entry<__bf16, __bf16, 128, 128, 64, 2, 2, false, true>("elemA_bf16_128x128x64_w2x2"),
      make_entry<__bf16, __bf16, 128, 128, 64, 2, 2, true, false>("elemB_bf16_128x128x64_w2x2"),
      make_entry<__bf16, __bf16, 128, 128, 64, 2, 2, false, false>("elemAB_bf16_128x128x64_w2x2"),
      make_dma_entry<__bf16, __bf16, 256, 256, 32, 4, 2, 4, true>("dma_bf16_256x256x32_s4_w2x4_pp"),
      make_dma_entry<__bf16, __bf16, 256, 256, 32, 4, 4, 2, true>("dma_bf16_256x256x32_s4_w4x2_pp"),
      make_ws_entry<__bf16, __bf16, 256, 128, 32, 6, 2, 2>("ws_bf16_256x128x32_s6_w2x2"),
      make_ws_entry<__bf16, __bf16, 128, 256, 32, 6, 2, 2>("ws_bf16_128x256x32_s6_w2x2"),
      make_ws_entry<__bf16, __bf16, 256, 128, 32, 4, 2, 2>("ws_bf16_256x128x32_s4_w2x2"),
      make_dma_entry<__bf16, __bf16, 256, 256, 64, 2, 2, 4, false, true>("dma_bf16_256x256x64_s2_w2x4_sk"),
      // few-row problems (split over K): A stored M x K only; four waves, or eight (two per SIMD)
      make_dma_entry<__bf16, __bf16, 64, 128, 64, 3, 2, 2>("dma_bf16_64x128x64_s3_w2x2"),
      make_dma_entry<__bf16, __bf16, 64, 128, 64, 4, 2, 4>("dma_bf16_64x128x64_s4_w2x4"),
  };
  *n = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace mg
