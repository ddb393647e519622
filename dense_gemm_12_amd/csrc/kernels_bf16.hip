// bf16-input GEMM configurations: v_mfma_f32_16x16x32_bf16, fp32 accumulate, output
// bf16 or fp32.  The 256 x 256 tiles of four waves (256 accumulators per lane,
// held in AGPRs) are instantiated here; every other configuration comes from
// kernels_bf16_vgpr.hip.
#include <vector>

#include "kernels_inst.hpp"

namespace mg {

const KernelEntry *entries_bf16(int *n) {
  static const std::vector<KernelEntry> table = [] {
    int m = 0;
    const KernelEntry *v = entries_bf16_vgpr(&m);
    std::vector<KernelEntry> t(v, v + m);
    // positions 2 and 6 keep the configuration ids of a single table
    t.insert(t.begin() + 2,
        make_dma_entry<__bf16, __bf16, 256, 256, 64, 2, 2, 2>("dma_bf16_256x256x64_s2_w2x2"));
    t.insert(t.begin() + 6,
        make_entry<__bf16, __bf16, 256, 256, 64, 2, 2, true, true>("mfma_bf16_256x256x64_w2x2"));
    return t;
  }();
  *n = (int)table.size();
  return table.data();
}

}  // namespace mg
