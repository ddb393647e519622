// Instantiation helpers: expand one tile configuration over the four storage
// layouts and the output types of an input type.
#pragma once
#include "gemm_dma_kernel.hpp"
#include "gemm_kernel.hpp"
#include "gemm_valu_kernel.hpp"

namespace mg {

// Workgroups of a kernel that fit on one CU at once (registers, LDS and
// waves together), as the HIP runtime computes it for the current device.
template <typename Kernel>
int occupancy_of(Kernel k, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, threads, 0) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the caller's next HIP call
    return -1;
  }
  return n;
}
template <class Tile> int occupancy_tile() { return occupancy_of(gemm_kernel<Tile>, Tile::NT); }
template <class Tile> int occupancy_dma_tile() { return occupancy_of(gemm_dma_kernel<Tile>, Tile::NT); }
template <class Tile> int occupancy_valu_tile() { return occupancy_of(gemm_valu_kernel<Tile>, Tile::NT); }

template <class Tile>
hipError_t launch_tile(const GemmParams &p, hipStream_t s) {
  hipLaunchKernelGGL(gemm_kernel<Tile>, dim3(p.tiles_m * p.tiles_n * p.splits), dim3(Tile::NT), 0, s, p);
  return hipGetLastError();
}

template <typename TI, typename TO, int BM, int BN, int BK, int WM, int WN, bool AV, bool BV>
struct LayoutSet {
  template <bool AKC, bool BKC>
  using T = GemmTile<TI, TO, BM, BN, BK, WM, WN, AKC, BKC, AV, BV>;
  static void fill(LaunchFn (&f)[2][2]) {
    f[0][0] = &launch_tile<T<false, false>>;
    f[0][1] = &launch_tile<T<false, true>>;
    f[1][0] = &launch_tile<T<true, false>>;
    f[1][1] = &launch_tile<T<true, true>>;
  }
};

// TI: input type; TO16: the 16-bit output type (ignored for fp32 inputs).
template <typename TI, typename TO16, int BM, int BN, int BK, int WM, int WN, bool AV, bool BV>
KernelEntry make_entry(const char *name) {
  KernelEntry e{};
  e.name = name;
  e.bm = BM;
  e.bn = BN;
  e.bk = BK;
  e.a_vec = AV;
  e.b_vec = BV;
  e.kind = 0;
  LayoutSet<TI, float, BM, BN, BK, WM, WN, AV, BV>::fill(e.fn[1]);
  if constexpr (sizeof(TI) == 4) {
    LayoutSet<TI, float, BM, BN, BK, WM, WN, AV, BV>::fill(e.fn[0]);
  } else {
    LayoutSet<TI, TO16, BM, BN, BK, WM, WN, AV, BV>::fill(e.fn[0]);
  }
  using Rep = typename LayoutSet<TI, float, BM, BN, BK, WM, WN, AV, BV>::template T<true, true>;
  e.threads = Rep::NT;
  e.lds_bytes = 2 * Rep::STAGE_BYTES;
  e.occupancy = &occupancy_tile<Rep>;
  return e;
}

template <class Tile>
hipError_t launch_dma_tile(const GemmParams &p, hipStream_t s) {
  const int grid = p.sk_grid > 0 ? p.sk_dp_tiles + p.sk_grid : p.tiles_m * p.tiles_n * p.splits;
  hipLaunchKernelGGL(gemm_dma_kernel<Tile>, dim3(grid), dim3(Tile::NT), 0, s, p);
  return hipGetLastError();
}

template <typename TI, typename TO, int BM, int BN, int BK, int ST, int WM, int WN, bool PP, bool SK = false>
struct DmaLayoutSet {
  template <bool AKC, bool BKC>
  using T = DmaTile<TI, TO, BM, BN, BK, ST, WM, WN, AKC, BKC, PP, SK>;
  // a layout whose operand slices have no supported LDS layout (e.g. a
  // k-major operand of fewer than 128 16-bit rows) is left null
  template <bool AKC, bool BKC>
  static LaunchFn fn() {
    constexpr int NW = WM * WN, ES = sizeof(TI);
    if constexpr (dma_operand_ok<BM, BK, AKC, NW, ES>() && dma_operand_ok<BN, BK, BKC, NW, ES>())
      return &launch_dma_tile<T<AKC, BKC>>;
    else
      return nullptr;
  }
  static void fill(LaunchFn (&f)[2][2]) {
    f[0][0] = fn<false, false>();
    f[0][1] = fn<false, true>();
    f[1][0] = fn<true, false>();
    f[1][1] = fn<true, true>();
  }
};

// Direct-to-LDS configurations (16-bit inputs, 16-byte-loadable operands).
template <typename TI, typename TO16, int BM, int BN, int BK, int ST, int WM, int WN, bool PP = false,
          bool SK = false>
KernelEntry make_dma_entry(const char *name) {
  KernelEntry e{};
  e.name = name;
  e.bm = BM;
  e.bn = BN;
  e.bk = BK;
  e.a_vec = true;
  e.b_vec = true;
  e.kind = 1;
  e.sk = SK;
  DmaLayoutSet<TI, float, BM, BN, BK, ST, WM, WN, PP, SK>::fill(e.fn[1]);
  DmaLayoutSet<TI, TO16, BM, BN, BK, ST, WM, WN, PP, SK>::fill(e.fn[0]);
  using Rep = typename DmaLayoutSet<TI, float, BM, BN, BK, ST, WM, WN, PP, SK>::template T<true, true>;
  e.threads = Rep::NT;
  e.lds_bytes = ST * Rep::STAGE_BYTES;
  e.occupancy = &occupancy_dma_tile<Rep>;
  return e;
}

template <typename TI, typename TO, int BM, int BN, int BK, int ST, int CWM, int CWN>
struct WsLayoutSet {
  template <bool AKC, bool BKC>
  using T = WsTile<TI, TO, BM, BN, BK, ST, CWM, CWN, AKC, BKC>;
  static void fill(LaunchFn (&f)[2][2]) {
    f[0][0] = &launch_dma_tile<T<false, false>>;
    f[0][1] = &launch_dma_tile<T<false, true>>;
    f[1][0] = &launch_dma_tile<T<true, false>>;
    f[1][1] = &launch_dma_tile<T<true, true>>;
  }
};

// Producer/consumer configurations (16-bit inputs, 16-byte-loadable operands).
template <typename TI, typename TO16, int BM, int BN, int BK, int ST, int CWM, int CWN>
KernelEntry make_ws_entry(const char *name) {
  KernelEntry e{};
  e.name = name;
  e.bm = BM;
  e.bn = BN;
  e.bk = BK;
  e.a_vec = true;
  e.b_vec = true;
  e.kind = 1;
  WsLayoutSet<TI, float, BM, BN, BK, ST, CWM, CWN>::fill(e.fn[1]);
  WsLayoutSet<TI, TO16, BM, BN, BK, ST, CWM, CWN>::fill(e.fn[0]);
  using Rep = typename WsLayoutSet<TI, float, BM, BN, BK, ST, CWM, CWN>::template T<true, true>;
  e.threads = Rep::NT;
  e.lds_bytes = ST * Rep::STAGE_BYTES;
  e.occupancy = &occupancy_dma_tile<Rep>;
  return e;
}

template <class Tile>
hipError_t launch_valu_tile(const GemmParams &p, hipStream_t s) {
  hipLaunchKernelGGL(gemm_valu_kernel<Tile>, dim3(p.tiles_m * p.tiles_n * p.splits), dim3(Tile::NT), 0, s,
                     p);
  return hipGetLastError();
}

// fp32 on the vector ALUs (kind 2): every layout, fp32 C only.
template <int BM, int BN, int BK>
KernelEntry make_valu_entry(const char *name) {
  KernelEntry e{};
  e.name = name;
  e.bm = BM;
  e.bn = BN;
  e.bk = BK;
  e.a_vec = true;
  e.b_vec = true;
  e.kind = 2;
  for (int c = 0; c < 2; ++c) {
    e.fn[c][0][0] = &launch_valu_tile<ValuTile<BM, BN, BK, false, false>>;
    e.fn[c][0][1] = &launch_valu_tile<ValuTile<BM, BN, BK, false, true>>;
    e.fn[c][1][0] = &launch_valu_tile<ValuTile<BM, BN, BK, true, false>>;
    e.fn[c][1][1] = &launch_valu_tile<ValuTile<BM, BN, BK, true, true>>;
  }
  using Rep = ValuTile<BM, BN, BK, true, true>;
  e.threads = Rep::NT;
  e.lds_bytes = 2 * Rep::STAGE_BYTES;
  e.occupancy = &occupancy_valu_tile<Rep>;
  return e;
}

}  // namespace mg
